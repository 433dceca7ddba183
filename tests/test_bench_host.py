"""Host logic of bench.py that runs without a GPU: the source digest that ties
the committed rocprofv3 counters to the kernels they were taken from (bench
reports the counted HBM traffic only while it matches)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_tokens_drop_comments_keep_literals():
    src = ('int a;  // note\n/* block\n comment */ const char* s = "// not a comment";\n'
           "char c = '/'; char q = '\\''; int d; /* tail */")
    assert bench._code_tokens(src) == (
        "int a; const char* s = \"// not a comment\"; char c = '/'; char q = '\\''; int d;")


def test_code_tokens_ignore_comment_reflow_but_not_code():
    a = "// one line\nint f(int x) { return x + 1; }\n"
    b = "// one\n// two lines\n\nint f(int x)   {\n  return x + 1;\n}\n"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_tokens(a) == bench._code_tokens(b)
    assert bench._code_tokens(a) != bench._code_tokens(c)



def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")


def test_ingest_counters_scales_by_the_copy_and_keeps_provenance(tmp_path, monkeypatch):
    import json
    out = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(out))
    monkeypatch.setattr(bench, "WORKLOADS", ("square",))
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    # the copy of 256 MiB reads 2 x its size by this counter: factor 0.5
    _csv(str(tmp_path / "pmc_fetch_square" / "run_counter_collection.csv"), hdr,
         [["copyBuffer", 1 << 20, "FETCH_SIZE", 2 * 256 * 1024],
          ["gemm_dma_kernel", 256, "FETCH_SIZE", 400000],
          ["gemm_dma_kernel", 256, "FETCH_SIZE", 410000],
          ["gemm_dma_kernel", 256, "FETCH_SIZE", 390000]])
    _csv(str(tmp_path / "pmc_write_square" / "run_counter_collection.csv"), hdr,
         [["copyBuffer", 1 << 20, "WRITE_SIZE", 256 * 1024],
          ["gemm_dma_kernel", 256, "WRITE_SIZE", 32768]])
    (tmp_path / "provenance.json").write_text(json.dumps({"taken": "2026-12-02", "gpu": "x"}))
    e = bench.ingest_counters(str(tmp_path))["square"]
    assert e["fetch_factor"] == 0.5 and e["fetch_bytes_per_launch"] == 400000 * 1024 // 2
    assert e["write_bytes_per_launch"] == 32768 * 1024
    assert e["provenance"] == {"taken": "2026-12-02", "gpu": "x"}
    got = bench.committed_counters("square")
    assert got is not None and bench.counters_entry(got)["taken"] == "2026-12-02"


def test_ingest_counters_sums_the_kernels_of_a_step(tmp_path, monkeypatch):
    # the split-K streaming step is two kernels: their medians add up
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "counters.json"))
    monkeypatch.setattr(bench, "WORKLOADS", ("skinny",))
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    for cn, c in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        _csv(str(tmp_path / f"pmc_{cn}_skinny" / "run_counter_collection.csv"), hdr,
             [["copyBuffer", 1 << 20, c, 256 * 1024],
              ["gemm_skinny_split_kernel", 512, c, 1000], ["skinny_split_reduce_kernel", 64, c, 10],
              ["gemm_skinny_split_kernel", 512, c, 1002], ["skinny_split_reduce_kernel", 64, c, 12],
              ["gemm_skinny_split_kernel", 512, c, 998], ["skinny_split_reduce_kernel", 64, c, 11]])
    e = bench.ingest_counters(str(tmp_path))["skinny"]
    assert e["fetch_bytes_per_launch"] == (1000 + 11) * 1024
    assert e["bytes_per_launch"] == 2 * (1000 + 11) * 1024
    assert "skinny_split_reduce_kernel" in e["kernel"]
