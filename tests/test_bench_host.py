"""Host-side pieces of bench.py: the one-GPU guard, the chain slicing and the
sharded oracle baseline's worker protocol (no GPU needed)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_chain_slice_takes_whole_sequences():
    shape = synth.C3
    inp = synth.chain_inputs(shape, config=3)
    sl = bench.chain_slice(inp, shape, 3, 2)
    assert sl["scores"].shape == (2,) + inp["scores"].shape[1:]
    np.testing.assert_array_equal(sl["scores"], inp["scores"][3:5])
    np.testing.assert_array_equal(sl["attn_proj"], inp["attn_proj"][3 * shape.seq:5 * shape.seq])
    np.testing.assert_array_equal(sl["gamma1"], inp["gamma1"])          # parameters stay whole


def test_sharded_oracle_baseline_runs_every_worker():
    r = bench.cpu_baseline_sharded(synth.C3, seconds=0.2)
    nseq = synth.C3.tokens // synth.C3.seq
    per = -(-nseq // min(len(os.sched_getaffinity(0)), nseq))          # sequences per worker
    assert r["cores"] == len(range(0, nseq, per))
    assert r["value"] > 0 and r["tokens_per_s"] > 0


def test_counter_staleness_hash_ignores_comments_only():
    """The stored counters stay valid across comment edits of the dominant
    kernel's sources and become stale on any code edit."""
    code = "int f(int a) {  // add one\n    return a + 1;  /* done */\n}\n"
    assert bench.code_text(code) == bench.code_text("// header\nint f(int a) {\n\n  return a + 1;\n}\n")
    assert bench.code_text(code) != bench.code_text(code.replace("a + 1", "a + 2"))
    assert bench.code_text("/* a\n multi-line\n comment */ x = 1;") == "x = 1;"


def test_cpu_baseline_reports_each_operator():
    r = bench.cpu_baseline(synth.C3, synth.DROPOUT_P, synth.DROPOUT_SEED, synth.LN_EPS, min_seconds=0.1,
                           max_seconds=5.0)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0
    _, counts, _ = bench.chain_bytes(512, synth.C3.hidden, synth.C3.ffn, synth.C3.heads, synth.C3.seq)
    assert set(r["per_operator"]) == set(counts)
    assert all(v["ms_per_call"] > 0 and v["GB/s"] > 0 for v in r["per_operator"].values())
    other = r["other_configs"]
    assert set(other) == {"transformer_big_chain", "embedding_fwd", "embedding_bwd", "adam_workspace_step"}
    assert all(v["GB/s"] > 0 for v in other.values())


def test_same_size_copy_covers_every_row():
    """Every row whose traffic the counters summary reports also gets a
    same-size copy reference (the bench passes other_rows_bytes() to it)."""
    rows = bench.other_rows_bytes()
    for row, _, _, _ in bench.ROW_KERNELS:
        assert row in rows and rows[row] > 0
    for key in ("tiny_chain C1 (3 calls)", "attention_softmax_fwd C2", "attention_softmax_bwd C2"):
        assert rows[key] > 0


@pytest.mark.parametrize("steps,g", [(1000, 12), (200, 12), (12, 12), (5, 12), (1, 12), (0, 12), (1000, 1),
                                     (50, 4), (13, 6)])
def test_graph_chunks_cover_every_step_once(steps, g):
    chunks = bench.graph_chunks(steps, g)
    covered = [i + k for i, n in chunks for k in range(n)]
    assert covered == list(range(steps))
    assert all(1 <= n <= g for _, n in chunks)
    assert all(n == g for _, n in chunks[:-1])
    assert all(i % g == 0 for i, _ in chunks)


@pytest.mark.parametrize("steps,g", [(1000, 12), (200, 12), (1000, 1), (24, 1), (5, 12), (100000, 12)])
def test_live_samples_stay_bounded(steps, g):
    n_graphs = len(bench.graph_chunks(steps, g))
    every = bench.sample_every_graphs(n_graphs, g)
    samples = -(-n_graphs // every)
    assert every >= 1
    assert every * g < 32 + g                 # a sample at least every ~32 steps
    assert samples >= min(n_graphs, 24)       # enough samples for the mean
