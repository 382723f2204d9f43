"""The oracle and the byte accounting against the values the pages state
(fixtures in tests/golden/, each with its citation)."""
import numpy as np

import bench
import oracle
from golden_data import beam_candidates_example, hars_example, load


def test_hars_worked_example_counts():
    """Beam 2 x vocabulary 8: 16 candidates, 5 of them left to sort; the top-k
    of the survivors is the top-k of a full sort of all 16."""
    lp, k, candidates, survivors = hars_example()
    assert lp.size == candidates
    s, i, surv = oracle.hars_topk(lp, None, k, return_survivors=True)
    assert surv[0] == survivors
    flat = lp.reshape(-1).astype(np.float64)
    order = np.lexsort((np.arange(flat.size), -flat))[:k]       # value descending, then index
    np.testing.assert_array_equal(i[0], order)
    np.testing.assert_array_equal(s[0], lp.reshape(-1)[order])


def test_beam_candidates_hand_computed():
    """Candidates with beam scores: one float32 addition, rounded to nearest
    even, worked out by hand in the fixture (exact sums, a tie to even in each
    direction, an absorbed quarter spacing); the top two follow from them."""
    lp, bs, c_ref, k, ids_ref, scores_ref = beam_candidates_example()
    c = oracle.beam_candidates(lp, bs)
    assert c.dtype == np.float32 and c.shape == c_ref.shape
    np.testing.assert_array_equal(c.view(np.uint32), c_ref.view(np.uint32))
    s, i = oracle.hars_topk(lp, bs, k)
    np.testing.assert_array_equal(i, ids_ref)
    np.testing.assert_array_equal(s.view(np.uint32), scores_ref.view(np.uint32))


def test_fused_elementwise_traffic_matches_the_pages_count():
    """A fused element-wise chain reads each input once and writes its output
    once: for one input and one output that is the page's 2 x size(x), against
    6 x size(x) for three separate kernels.  The chain's algorithmic bytes
    follow the same rule (parameters vectors aside)."""
    d = load("fusion_traffic.txt")
    assert d["unfused_traffic"] == 2 * d["unfused_ops"]          # one read and one write per kernel
    tokens, hidden, ffn, heads, seq = 4096, 768, 3072, 12, 128
    per, _, _ = bench.chain_bytes(tokens, hidden, ffn, heads, seq)
    size = lambda elems: 2 * elems                               # fp16 storage  # noqa: E731
    # bias + ReLU + dropout: one activation in, one out (the page's shape)
    assert per["bias_relu_dropout"] - size(ffn) == d["fused_traffic"] * size(tokens * ffn)
    # bias + dropout + residual: two activations in, one out
    assert per["bias_dropout_residual"] - size(hidden) == (d["fused_traffic"] + 1) * size(tokens * hidden)
    # softmax forward: scores in, probabilities out
    e_s = tokens // seq * heads * seq * seq
    assert per["softmax_fwd"] == d["fused_traffic"] * size(e_s)
    # three unfused element-wise kernels over the FFN activation would move 3x the fused bytes
    assert d["unfused_traffic"] * size(tokens * ffn) == 3 * (per["bias_relu_dropout"] - size(ffn))
