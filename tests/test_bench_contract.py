"""The benchmark's host-side contract, without a GPU: a request for more than
one GPU exits with an explanation, and the counter traffic it reports comes
from a committed rocprofv3 summary only while the kernel sources are the ones
that summary was taken from."""
from __future__ import annotations

import glob
import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    msg = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def _write_summary(root, workload, sha, traffic):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"paged_decode_attn__{workload}__pmc.txt"), "w") as f:
        f.write(f"# header\ntraffic_bytes_per_launch: {traffic}\nsource_sha256: {sha}\n")


def test_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "attn_source_hash", lambda: "abc")
    _write_summary(str(tmp_path), "w_ok", "abc", 123456)
    _write_summary(str(tmp_path), "w_stale", "def", 654321)
    assert bench.measured_traffic("w_ok") == 123456
    assert bench.measured_traffic("w_stale") is None        # sources changed since
    assert bench.measured_traffic("w_missing") is None      # never profiled


def test_committed_summaries_are_well_formed():
    paths = glob.glob(os.path.join(ROOT, "profiles", "paged_decode_attn__*__pmc.txt"))
    assert paths
    for p in paths:
        fields = {}
        for line in open(p):
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        assert int(fields["traffic_bytes_per_launch"]) > 0, p
        assert len(fields["source_sha256"]) == 64, p
        workload = os.path.basename(p)[len("paged_decode_attn__"):-len("__pmc.txt")]
        assert os.path.exists(p.replace("__pmc.txt", "__kernel_trace.txt")), workload


def test_source_hash_follows_code_not_comments():
    a = 'int f(int x) { return x + 1; }  // add one\n/* block\n comment */ const char* s = "//x";\n'
    b = '// a header\nint f(int x)   {\n    return x + 1;   /* same */ }\nconst char* s = "//x";\n'
    c = 'int f(int x) { return x + 2; }\nconst char* s = "//x";\n'
    d = 'int f(int x) { return x + 1; }\nconst char* s = "/x";\n'
    assert bench.code_tokens(a) == bench.code_tokens(b)          # comments, layout
    assert bench.code_tokens(a) != bench.code_tokens(c)          # code
    assert bench.code_tokens(a) != bench.code_tokens(d)          # string literal contents
    assert bench.code_tokens("char q = '\"'; // c") == "char q = '\"';"
