"""Host-side pieces of bench.py: the one-GPU guard, the chain slicing and the
sharded oracle baseline's worker protocol (no GPU needed)."""
import os
import subprocess
import sys

import numpy as np

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
