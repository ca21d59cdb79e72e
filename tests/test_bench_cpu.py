"""Host logic of bench.py (CPU only): the algorithmic work each kernel's
roofline divides by, the rule that counter traffic comes only from a summary
of the current sources, and the one-GPU guard."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from workload import configs  # noqa: E402


def test_algorithmic_work_at_the_4k_layer():
    """Config 3 (T = 8192 tokens per rank, d_model 6144, 384 experts, top-8,
    latent 3072, expert hidden 1536, 2 shared experts of hidden 1536, 64 ranks)
    with 67,944 rows kept at receive over 3 waves and all 65,536 assignments
    kept at send (pool cap 1127): each figure worked out by hand from those
    dimensions, as the design notes' kernel table lists them."""
    sh = configs.get(3)
    w = bench.algorithmic_work(sh, [67944 / 3] * 3, send_kept=65536, send_cap=1127)
    # route: x [8192 x 6144] times [W_r ; W_d] [(384 + 3072) x 6144]
    assert w["route_gemm"] == ("flop", 2 * 8192 * 3456 * 6144) and w["route_gemm"][1] == 347_892_350_976
    # gate/up of a wave: 22,648 kept rows x 3072 (gate and up, 1536 each) x K = 3072
    assert w["expert_gate_up"] == ("flop", 427_466_686_464.0)
    # down of a wave: 22,648 rows x 3072 x K = 1536
    assert w["expert_down"] == ("flop", 213_733_343_232.0)
    # shared gate/up: 8192 x (2 experts x 2 x 1536) x 6144; up + shared down: 8192 x 6144 x (3072 + 2 x 1536)
    assert w["shared_gate_up"] == ("flop", 618_475_290_624)
    assert w["up_shared_down"] == ("flop", 618_475_290_624)
    # pack: z read once (8192 x 6144 B), 65,536 rows of 6144 B payload + 4 B id written, the ids of the
    # 64 x 1127 - 65,536 = 6592 empty slots, top-k ids read and slot_of written (8 B per assignment)
    assert w["pack"] == ("byte", 50_331_648 + 65536 * 6148 + 4 * 6592 + 8 * 65536)
    # combine: 65,536 returned rows of 6144 B read, weights and slots (8 B per assignment), c written
    assert w["combine"] == ("byte", 65536 * 6144 + 8 * 65536 + 50_331_648)


def _summary(root, kernel, workload, digest, value="123456"):
    d = root / "profiles"
    d.mkdir(exist_ok=True)
    (d / f"{kernel}_{workload}_pmc.txt").write_text(
        f"HBM-side traffic of {kernel}\nsource_digest: {digest}\nhbm_bytes_per_launch: {value}\n")


def test_counter_traffic_only_from_a_summary_of_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "0123456789abcdef")
    assert bench.committed_traffic("expert_gate_up", "w") is None  # no summary
    _summary(tmp_path, "expert_gate_up", "w", "0123456789abcdef")
    assert bench.committed_traffic("expert_gate_up", "w") == 123456.0
    _summary(tmp_path, "expert_gate_up", "w", "fedcba9876543210")  # taken from other sources
    assert bench.committed_traffic("expert_gate_up", "w") is None
    _summary(tmp_path, "expert_gate_up", "w", "0123456789abcdef", value="n/a")
    assert bench.committed_traffic("expert_gate_up", "w") is None


def test_source_digest_covers_every_library_source():
    """A change to any kernel or host source of the library changes the digest,
    so no counter summary outlives the code it was taken from."""
    csrc = os.path.join(ROOT, "grouped_expert_ffn_router_amd", "csrc")
    files = {os.path.join("grouped_expert_ffn_router_amd", "csrc", f) for f in os.listdir(csrc)
             if f.endswith((".hip", ".h"))}
    assert files <= set(bench.SOURCES)
    assert all(os.path.exists(os.path.join(ROOT, p)) for p in bench.SOURCES)
    d = bench.source_digest()
    assert len(d) == 16 and d == bench.source_digest()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads([l for l in r.stdout.splitlines() if l.startswith("{")][-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


@pytest.mark.parametrize("cfg", [2, 3, 4, 5, 6])
def test_every_benchmark_workload_has_committed_summaries(cfg):
    """Each workload's kernel trace and its dominant kernel's traffic summary
    are committed for the current sources."""
    w = configs.get(cfg).name
    trace = os.path.join(ROOT, "profiles", f"layer_kernels_{w}_trace.md")
    assert os.path.exists(trace) and bench.source_digest() in open(trace).read()
    dominant = "expert_gate_up" if configs.get(cfg).layer == "full" else "route_gemm"
    assert bench.committed_traffic(dominant, w) is not None
