"""Host-side logic of the benchmark (no GPU): the source hash that marks a
committed counter summary stale."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


SRC = """// header comment
#include "x.h"
/* a block
   comment */
__global__ void k(float* p) {   // trailing comment
    p[0] = 1.0f;
}
"""


def test_code_text_ignores_comments_and_blank_space():
    edited = SRC.replace("header comment", "another header").replace("trailing comment", "")
    edited = edited.replace("    p[0]", "        p[0]") + "\n\n"
    assert bench.code_text(edited) == bench.code_text(SRC)


def test_code_text_sees_code_changes():
    assert bench.code_text(SRC.replace("1.0f", "2.0f")) != bench.code_text(SRC)
    assert bench.code_text(SRC.replace("p[0]", "p[1]")) != bench.code_text(SRC)


def test_committed_counter_summaries_name_known_kernels():
    import glob
    import json
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.json")):
        with open(path) as fh:
            rec = json.load(fh)
        assert rec["kernel"] in bench.KERNEL_SOURCES, path
        assert len(rec["source_sha"]) == 16, path
