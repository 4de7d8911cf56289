"""Host logic of bench.py: the byte accounting of a step, the one-GPU guard and
the traffic-profile gating.  No GPU is used."""
import os
import subprocess
import sys

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_direct_step_bytes_qwen3():
    cfg = W.get_config("qwen3_30b_a3b")
    TH = cfg.T * cfg.H * 2
    RH = cfg.R * cfg.H * 2
    total = sum(b for *_, b in bench.step_calls(cfg))
    assert total == 4 * TH + 5 * RH == 738_197_504


@pytest.mark.parametrize("name", ["tiny", "qwen3_30b_a3b", "deepseek_v3"])
def test_staged_step_adds_the_send_buffer_traffic(name):
    """Staged = direct + one more token-row read (the row-free dot re-reads g)
    + 8 send-buffer passes (send, expand, reduce, merge; forward and backward)."""
    cfg = W.get_config(name)
    n_send = cfg.T * 2 + 5
    TH = cfg.T * cfg.H * cfg.esize
    NS = n_send * cfg.H * cfg.esize
    direct = sum(b for *_, b in bench.step_calls(cfg))
    staged = bench.step_calls(cfg, True, [n_send])
    assert sum(b for *_, b in staged) == direct + TH + 8 * NS
    assert bench.dominant_call(cfg, True) in [c[0] for c in staged]
    kinds = [c[1] for c in staged]
    assert kinds.count("send_x") == 1 and kinds.count("send_g") == 1 and kinds.count("dot_w") == 1


def test_staged_absorbed_step_has_three_passes_and_two_backwards():
    cfg = W.get_config("diffusion_gemma")
    calls = bench.step_calls(cfg, True, [10, 20, 30])
    names = [c[0] for c in calls]
    assert names.count("layout.0") == 1 and "replay_layout.2" in names and "replay_layout.1" not in names
    assert sum(1 for c in calls if c[1] == "dot_s") == 2
    assert bench.dominant_call(cfg, True) == "dispatch.0:expand"
    assert bench.dominant_call(cfg) == "dispatch.0"
    NS = {p: n * cfg.H * cfg.esize for p, n in enumerate([10, 20, 30])}
    for name, kind, p, b in calls:
        if kind.startswith("send"):
            assert b == cfg.T * cfg.H * cfg.esize + NS[p], name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("extra", [("--graph-steps", "2"),                         # without --graph
                                   ("--graph", "--graph-steps", "3"),              # 3 does not divide 200
                                   ("--graph", "--graph-steps", "4", "--warmup", "6"),
                                   ("--graph", "--graph-steps", "0")])
def test_graph_steps_must_divide_the_run(extra):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *extra],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--graph-steps" in r.stderr and not r.stdout


def test_traffic_is_reported_only_for_matching_sources(tmp_path, monkeypatch):
    """The counters stay valid while the dominant kernel, its launcher and
    the device helpers are unchanged; an edit elsewhere in the file keeps
    them, an edit to the kernel drops them."""
    cfg = W.get_config("qwen3_30b_a3b")
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "combine_moe_layout_04_amd" / "csrc"
    csrc.mkdir(parents=True)

    def source(kernel, launcher, body="  a.x = 1;", other="// other code"):
        return (f"{other}\ntemplate <int DT>\n__global__ __launch_bounds__(512) void {kernel}(Args a) {{\n{body}\n}}\n"
                f"\ntemplate <int DT>\nhipError_t {launcher}(Args a) {{\n  return 0;\n}}\n")

    (csrc / "row_kernels.hip").write_text(source("scatter_kernel", "go_scatter"))
    (csrc / "staged_kernels.hip").write_text(source("expand_kernel", "go_expand"))
    (csrc / "device_common.h").write_text("// helpers\n")
    (csrc / "pad_fill.h").write_text("// padding waves\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    hd, hs = bench.kernel_source_hash(False), bench.kernel_source_hash(True)
    (tmp_path / "profiles" / f"traffic_{cfg.name}.md").write_text(
        f"source_hash.dispatch: {hd}\ntraffic_bytes_per_launch.dispatch: 123\n"
        f"source_hash.dispatch:expand: {hs}\ntraffic_bytes_per_launch.dispatch:expand: 456\n")
    assert bench.traffic_from_profiles(cfg) == 123
    assert bench.traffic_from_profiles(cfg, True) == 456
    (csrc / "row_kernels.hip").write_text(source("scatter_kernel", "go_scatter", other="// edited elsewhere"))
    assert bench.traffic_from_profiles(cfg) == 123
    (csrc / "staged_kernels.hip").write_text(source("expand_kernel", "go_expand", body="  a.x = 2;"))
    assert bench.traffic_from_profiles(cfg) == 123
    assert bench.traffic_from_profiles(cfg, True) is None
    (csrc / "pad_fill.h").write_text("// padding waves, changed\n")
    assert bench.traffic_from_profiles(cfg) is None


def test_sources_hash_names_the_code(tmp_path, monkeypatch):
    """The result line's sources hash changes with any library source."""
    csrc = tmp_path / "combine_moe_layout_04_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "include").mkdir()
    (tmp_path / "include" / "moe_layout.h").write_text("// header\n")
    (csrc / "a.hip").write_text("// a\n")
    (csrc / "notes.txt").write_text("not a source\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.sources_hash()
    (csrc / "notes.txt").write_text("changed, still not a source\n")
    assert bench.sources_hash() == h0
    (csrc / "a.hip").write_text("// a, changed\n")
    assert bench.sources_hash() != h0


@pytest.mark.parametrize("nsets,warmup,steps", [(18, 5, 20), (18, 20, 200), (5, 10, 50), (3, 0, 7), (1, 2, 3)])
def test_rotation_touches_every_set_first_and_keeps_timed_sets_cold(nsets, warmup, steps):
    """Set-up runs every buffer set once before anything is timed, and every
    timed step's set was last used exactly nsets - 1 steps before it."""
    o = bench.rotation(nsets, warmup, steps)
    assert sorted(o["setup"]) == list(range(nsets))
    seq = o["setup"] + o["warmup"] + o["headline"] + o["event"]
    t0 = len(o["setup"]) + len(o["warmup"])
    last = {}
    for i, j in enumerate(seq):
        if i >= t0:
            assert j in last                          # never first touched in a timed phase
            assert i - last[j] == nsets, (i, j, last[j])  # nsets - 1 other steps in between
        last[j] = i
