"""bench.py's command-line contract on the CPU: one GPU only (a message and a
non-zero exit for --gpus N > 1), and every workload it names is accepted by
the parser and has synthetic inputs."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_workloads_have_inputs():
    sys.path.insert(0, ROOT)
    import bench
    from late_interaction_retrieval_amd import inputs
    old = sys.argv
    try:
        sys.argv = ["bench.py", "--workload", "chamfer_batch"]
        assert bench.parse().workload == "chamfer_batch"
    finally:
        sys.argv = old
    for name in inputs.WORKLOADS:
        w = inputs.make(name, B=4, Nq=2)  # the recipe at a small size
        assert w["Q"].shape[0] == 2 and w["cu_seqlens"].shape == (5,)
    for name in inputs.CHAMFER_WORKLOADS:
        w = inputs.make_chamfer(name, Bt=2, N=16, M=8)
        assert w["P"].shape == (2, 16, 3) and w["Q"].shape == (2, 8, 3)


def test_default_line_is_the_colpali_headline_with_every_config():
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        assert bench.parse().workload == "all"
    finally:
        sys.argv = old
    assert bench.HEADLINE == "colpali_fwd"
    assert set(bench.ALL_CONFIGS) == {"colbert_tiny", "colbert_rerank_varlen", "colbert_rerank_padded",
                                      "colpali_fwd", "contrastive_train", "int8_varlen"}


def test_cpu_baseline_names_the_host():
    sys.path.insert(0, ROOT)
    import bench
    from late_interaction_retrieval_amd import inputs
    w = inputs.make("colbert_rerank_varlen", B=3, Nq=2)
    c = bench.cpu_baseline(w, 0.01)
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["nproc"] >= 1
    assert "cpu_model" in c and c["value"] > 0 and "documents" in c["sample"]
