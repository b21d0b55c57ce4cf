"""Host-side logic of bench.py (no GPU): the source hash that keys measured
traffic to the kernels it was measured on."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import bench  # noqa: E402


def test_source_text_drops_comments_and_blank_lines():
    src = "int a; // note\n\n/* block\n comment */ int b;  \n  // only a comment\nint c; /* x */ int d;\n"
    assert bench.source_code_text(src) == "int a;\n int b;\nint c;  int d;"


def test_hash_ignores_comments_but_not_code():
    files = {f: open(os.path.join(bench.ROOT, "paged_kv_cache_419_amd", "csrc", f)).read()
             for call in bench.CALL_SOURCES for f in bench.CALL_SOURCES[call] + bench.SHARED_SOURCES}
    for call in bench.CALL_SOURCES:
        base = bench.kernel_sources_sha(call, files.__getitem__)
        assert base == bench.kernel_sources_sha(call)
        target = bench.CALL_SOURCES[call][0]
        commented = dict(files)
        commented[target] = "// a new comment\n\n" + files[target].replace("\n", "  /* c */\n", 3)
        assert bench.kernel_sources_sha(call, commented.__getitem__) == base
        changed = dict(files)
        changed[target] = files[target] + "\nstatic int added_line;\n"
        assert bench.kernel_sources_sha(call, changed.__getitem__) != base
