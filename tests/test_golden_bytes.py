"""The byte model used for the roofline reproduces the pages' worked example
(tests/golden/state_bytes.txt)."""
import os

from hyper_connections_amd import traffic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "state_bytes.txt")


def rows():
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            yield tuple(int(v) for v in line.split())


def test_state_bytes_worked_example():
    got = list(rows())
    assert len(got) == 3
    for n, d, s, tokens, expect in got:
        assert traffic.state_bytes(n, d, s, tokens) == expect
    # "a 4x increase, and 48 KB more per token per boundary"
    one, four = traffic.state_bytes(1, 8192, 2), traffic.state_bytes(4, 8192, 2)
    assert four == 4 * one and four - one == 48 * 1024


def test_layer_bytes_are_14_state_units_at_n4():
    """pre reads the state and writes one stream; post reads state and F and
    writes the state: (n+1) + (2n+1) = 3n+2 hidden-width vectors per token."""
    n, d, s = 4, 4096, 2
    assert traffic.pre_bytes(n, d, s) + traffic.post_bytes(n, d, s) == 14 * d * s == 114688


def test_backward_bytes_count_each_row_moved():
    """Backward rows per token at n = 4: post reads dH', H and F (2n+1) and
    writes dH and dF (n+1), or only dF when the pre gradient forms dH; pre
    reads du, H and dH_in or dH' (2n+1) and writes dH (n).  Folding removes
    exactly the n rows of post's dH write from the layer."""
    n, d, s = 4, 4096, 2
    rec = traffic.record_bytes(n)
    assert traffic.post_bwd_bytes(n, d, s) == (3 * n + 2) * d * s + rec == 114688 + rec
    assert traffic.post_bwd_bytes(n, d, s, h_grad=False) == (2 * n + 2) * d * s + rec == 81920 + rec
    assert traffic.pre_bwd_bytes(n, d, s, True) == (3 * n + 1) * d * s + rec == 106496 + rec
    unfolded = traffic.post_bwd_bytes(n, d, s) + traffic.pre_bwd_bytes(n, d, s, True)
    folded = traffic.post_bwd_bytes(n, d, s, h_grad=False) + traffic.pre_bwd_bytes(n, d, s, True)
    assert unfolded - folded == n * d * s


def test_weight_producer_factors_bytes():
    """The dynamic layer's backward per token at n = 4, d = 4096, bf16, one
    pass per boundary.  With the producer's gradient added in place: dalpha
    alone (H and du, n + 1 rows), the producer (H, dH in, dH out: 3n rows)
    and the boundary (3n + 3 rows): 32 rows.  As its factors: the producer
    reads H (n rows) and writes dhbar (d fp32, two bf16 rows) and 2n
    coefficients; the boundary reads them too: 28 rows, 12.4% fewer bytes."""
    n, d, s = 4, 4096, 2
    rec = traffic.record_bytes(n)
    coef = 4 * 2 * n
    assert traffic.weights_bwd_terms_bytes(n, d, s) == n * d * s + 4 * d + coef + 2 * rec == 49376
    assert (traffic.post_pre_bwd_terms_bytes(n, d, s)
            == traffic.post_pre_bwd_bytes(n, d, s, True) + 4 * d + coef == 139680)
    alone = traffic.pre_records_bytes(n, d, s)
    in_place = alone + traffic.weights_bwd_bytes(n, d, s) + traffic.post_pre_bwd_bytes(n, d, s, True)
    factors = (alone + traffic.weights_bwd_terms_bytes(n, d, s)
               + traffic.post_pre_bwd_terms_bytes(n, d, s))
    assert in_place == 262816 and factors == 230112
    assert in_place - factors == 4 * d * s - 2 * coef
