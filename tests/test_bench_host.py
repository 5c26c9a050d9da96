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
    paths = (glob.glob(os.path.join(ROOT, "profiles", "*_counters.json")) +
             glob.glob(os.path.join(ROOT, "profiles", "*_mfma.json")))
    assert paths
    for path in paths:
        with open(path) as fh:
            rec = json.load(fh)
        assert rec["kernel"] in bench.KERNEL_SOURCES, path
        assert len(rec["source_sha"]) == 16, path


def test_committed_drift_summary_is_within_its_bound():
    import json
    with open(os.path.join(ROOT, "profiles", "chain-bf16_drift.json")) as fh:
        rec = json.load(fh)
    assert len(rec["rows"]) == rec["layers"] == 78
    drift = [r["drift_vs_bf16_storing_fp64"] for r in rec["rows"]]
    assert max(drift) == rec["max_drift_vs_bf16_storing_fp64"] <= rec["drift_bound"]


def test_kernel_match_tells_the_kernels_apart():
    """Trace and counter rows are attributed by the whole kernel identifier
    and, where one template serves two entry points, its last argument."""
    ns = "void hc::(anonymous namespace)::"
    tail = "(unsigned char const*, float const*)"
    names = {
        "pre_mix_backward": ns + "pre_bwd_kernel<4, hc::bf16_t, 1, true, true, true>" + tail,
        "pre_mix_records": ns + "pre_bwd_kernel<4, hc::bf16_t, 1, true, false, false>" + tail,
        "post_pre_mix_backward": ns + "post_pre_bwd_kernel<4, hc::bf16_t, 1, true, false>" + tail,
        "post_pre_mix_backward_terms": ns + "post_pre_bwd_kernel<4, hc::bf16_t, 1, true, true>" + tail,
        "weights_backward_stream": ns + "wgrad_mfma_kernel<4, true, false>" + tail,
        "weights_backward_terms_stream": ns + "wgrad_mfma_kernel<4, false, true>" + tail,
        "post_mix_backward": ns + "post_bwd_kernel<4, hc::bf16_t, 1, false, false>" + tail,
        "pre_mix": ns + "pre_mix_kernel<4, hc::bf16_t, 1>" + tail,
        "post_pre_mix": ns + "post_pre_mix_kernel<4, hc::bf16_t, 1>" + tail,
        "post_weights_pre_mix": ns + "post_weights_kernel<4, hc::bf16_t, 4, 1, true, true>" + tail,
        "post_mix_weights": ns + "post_weights_kernel<4, hc::bf16_t, 4, 1, true, false>" + tail,
    }
    for kernel, name in names.items():
        hits = [k for k in names if bench.kernel_match(k, name)]
        assert hits == [kernel], (kernel, hits)
