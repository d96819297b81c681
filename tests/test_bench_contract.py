"""CPU checks of bench.py's contract that need no GPU: more than one GPU is
refused with a message (the build runs one rank's shard on one MI355X), and
the committed counter summaries parse (their traffic is reported only while
their source hash matches the kernels)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_summaries_parse():
    sys.path.insert(0, ROOT)
    import bench
    # each GEMM summary covers every launch of its workload's timed step (bench.py's kernel
    # names; bench.py --workload picks the workload); the decode summary the whole one-token call
    cases = [(f"gemm_hbm_traffic_{w}.md", bench.GEMM_SOURCES, k)
             for w in ("gpt3_train_t8", "llama_7b_train_t2", "llama3_70b_prefill_t4")
             for k in ("up_act", "down", "reduce_y", "down_bwd", "up_bwd", "reduce_dx")]
    cases.append(("gemv_hbm_traffic_llama3_70b_decode_t4.md", bench.GEMV_SOURCES, "decode"))
    for summary, files, kernel in cases:
        path = os.path.join(ROOT, "profiles", summary)
        assert os.path.exists(path), summary
        with open(path) as fh:
            line = [ln for ln in fh if ln.startswith("traffic_json: ")]
        assert len(line) == 1, summary
        assert kernel in json.loads(line[0][len("traffic_json: "):])["kernels"], (summary, kernel)
        info = bench.counter_traffic(summary, files, kernel)
        # None only when the kernels changed after the counters were taken
        if info is not None:
            assert info["bytes"] > 0 and info["algorithmic_bytes"] > 0


def test_source_hash_ignores_comments_only():
    """The counter summaries are keyed to the kernels' code: comments and
    blank lines do not change the hash, any code (strings included) does."""
    import bench
    a = 'int f() { return 1; }  // one\n/* block\n comment */\nconst char* s = "x // not a comment";\n'
    b = 'int f() { return 1; }\n\n// another comment\nconst char* s = "x // not a comment";   \n'
    c = 'int f() { return 2; }\nconst char* s = "x // not a comment";\n'
    d = 'int f() { return 1; }\nconst char* s = "x // still not one";\n'
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only(c)
    assert bench.code_only(a) != bench.code_only(d)
    assert "/*" not in bench.code_only(a) and "// one" not in bench.code_only(a)
