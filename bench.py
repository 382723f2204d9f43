"""Throughput of the fused non-GEMM chain of one BERT-base layer on one MI355X.

One step is one pass of the layer's non-GEMM hot path over a 4096-token batch
(32 sequences x 128, hidden 768, 12 heads, FFN 3072, fp16 storage, fp32
arithmetic, dropout 0.1):

  softmax fwd [32,12,128,128] -> bias+dropout+residual -> LayerNorm [4096,768]
  (one fused call) -> bias+ReLU+dropout [4096,3072] -> the fused block again
  -> LayerNorm bwd input gradients x2 -> both LayerNorms' parameter gradients
  (one call) -> softmax bwd

Inputs are synthetic (seeded, shaped like the layer) and resident in HBM before
the timed region.  R independent buffer sets (> 2 GB in total; 12 by default,
one per layer of BERT-base) are rotated so that no step finds its tensors in
the 256 MB Infinity Cache.  The timed steps are replayed as HIP graphs of G
consecutive steps (one step per set in turn; G = R by default, a training
iteration's layers in one graph).  Every few timed graphs one is replayed
split around its first LayerNorm backward, the operator whose row kernel
takes the largest share of the step (two launches of it per step), which is
then called directly on the same stream with a pair of HIP events attached
to its row kernel's launch (hipExtLaunchKernel records them when the kernel
starts and ends): the events sample that kernel's duration live inside the
timed region (the roofline line).
The largest single launch, bias+ReLU+dropout, is reported beside it from the
cold per-kernel timing.

Output: one JSON line.  `value` is algorithmic chain bytes per second (the
fused-minimum bytes: every input read once, every output written once, the
dropout mask regenerated, not stored) and `tokens_per_s` the chain rate.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--graph-steps G] [--no-cpu] [--no-extra]
       python bench.py --summarize-counters FETCH.csv WRITE.csv   (writes profiles/)
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
# The dominant kernel: the one with the largest share of the chain's time --
# the LayerNorm backward's row kernel, launched twice per step.  The fused
# block's kernel (also twice per step) takes about as much time, a few percent
# more in the kernel trace, at a higher fraction of its roofline; the lower
# one is reported.
# (The largest single launch, bias+ReLU+dropout, is reported beside it.)
DOMINANT = "layernorm_bwd"
DOMINANT_SHAPE = "[4096,768]"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "layernorm_bwd_4096x768_counters.json")
KERNEL_SYMBOL = "ln_bwd_kernel"              # substring of the dominant kernel's symbol
LARGEST = "bias_relu_dropout"


# ---------------------------------------------------------------------------
# Algorithmic (fused-minimum) byte counts
# ---------------------------------------------------------------------------

def chain_bytes(tokens, hidden, ffn, heads, seq, fused=True):
    """Algorithmic bytes per call of every operator, calls per step, and the
    step's total.  fused: each bias+dropout+residual and the LayerNorm after
    it are one operator, which does not read its own sum back."""
    e_h, e_f = tokens * hidden, tokens * ffn
    e_s = (tokens // seq) * heads * seq * seq
    rows = tokens
    per = {
        "softmax_fwd": 4 * e_s,                                   # read x, write y
        "bias_dropout_residual": 6 * e_h + 2 * hidden,            # x, residual, out (+bias)
        "layernorm_fwd": 4 * e_h + 8 * rows + 4 * hidden,         # x, y, mean+rstd (+gamma, beta)
        # x, residual, z, y, mean+rstd (+bias, gamma, beta)
        "bias_dropout_residual_layernorm": 8 * e_h + 8 * rows + 6 * hidden,
        "bias_relu_dropout": 4 * e_f + 2 * ffn,                   # x, out (+bias)
        "layernorm_bwd": 6 * e_h + 8 * rows + 6 * hidden,         # dy, x, dx, stats, gamma, dgamma, dbeta
        # its two calls: the input gradient (row kernel) and the parameter gradients
        "layernorm_bwd_input": 6 * e_h + 8 * rows + 2 * hidden,
        "layernorm_bwd_params": 4 * hidden,
        "softmax_bwd": 6 * e_s,                                   # y, dy, dx
    }
    counts = {"softmax_fwd": 1, "bias_relu_dropout": 1, "layernorm_bwd": 2, "softmax_bwd": 1}
    if fused:
        counts["bias_dropout_residual_layernorm"] = 2
    else:
        counts.update(bias_dropout_residual=2, layernorm_fwd=2)
    total = sum(per[k] * counts[k] for k in counts)
    return per, counts, total


DOMINANT_SOURCES = ("layernorm.hip", "ls_common.hpp")


def code_text(src):
    """C++ source without its comments and blank-line or indentation changes:
    what the compiler sees of it, so that a comment edit does not make
    stored counters look stale.  (String literals are not parsed; a "//"
    inside one cuts the rest of that line for hashing, the same way each time.)"""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).strip() for ln in src.splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_hash():
    """Hash of the dominant kernel's sources (their code, not their comments),
    used to tell whether stored counters are stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "non_gemm_amd", "csrc")
    for name in DOMINANT_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# HIP events for the dominant kernel, handed to the library with
# ls_time_next_launch(): its launch records them itself (hipExtLaunchKernel),
# so each pair brackets that kernel's execution and nothing else.
# ---------------------------------------------------------------------------

class KernelEvents:
    HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")      # the runtime torch already loaded
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            for e in (a, b):
                if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.HIP_EVENT_DISABLE_SYSTEM_FENCE):
                    raise RuntimeError("hipEventCreateWithFlags failed")
            self.pairs.append((a, b))

    def arm(self, i, lib):
        """The next launch of this thread that goes through the timing hook records pair i."""
        if lib.ls_time_next_launch(self.pairs[i][0], self.pairs[i][1]) != 0:
            raise RuntimeError("ls_time_next_launch failed")

    def mean_us(self):
        tot = 0.0
        for a, b in self.pairs:
            ms = self.ct.c_float()
            if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b):
                raise RuntimeError("hipEventElapsedTime failed")
            tot += ms.value
        return tot / len(self.pairs) * 1e3

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


# ---------------------------------------------------------------------------
# GPU chain
# ---------------------------------------------------------------------------

class ChainSet:
    """Device buffers of one step, and its launches as (name, bytes, call)."""

    def __init__(self, torch, inputs, shape, lib, per_bytes, p, seed, eps, fused=True, batched_params=True):
        d = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
        self.torch = torch
        self.t = {k: d(v) for k, v in inputs.items()}
        t = self.t
        T, H, F = shape.tokens, shape.hidden, shape.ffn
        B, NH, L = shape.batch, shape.heads, shape.seq
        f16, f32 = torch.float16, torch.float32
        new = lambda *s, dt=f16: torch.empty(s, dtype=dt, device="cuda")  # noqa: E731
        t["probs"] = new(B, NH, L, L)
        t["dscores"] = new(B, NH, L, L)
        t["attn_out"] = new(T, H)
        t["ln1"] = new(T, H)
        t["ffn_act"] = new(T, F)
        t["ffn_out"] = new(T, H)
        t["ln2"] = new(T, H)
        t["dx1"] = new(T, H)
        t["dx2"] = new(T, H)
        for k in ("mean1", "rstd1", "mean2", "rstd2"):
            t[k] = new(T, dt=f32)
        for k in ("dg1", "db1", "dg2", "db2"):
            t[k] = new(H)
        ws = lib.ls_layernorm_bwd_workspace_bytes(T, H)
        t["ws1"] = torch.empty(ws, dtype=torch.uint8, device="cuda")
        t["ws2"] = torch.empty(ws, dtype=torch.uint8, device="cuda")
        P = {k: v.data_ptr() for k, v in t.items()}
        self.ptr = P
        S = torch.cuda.current_stream().cuda_stream
        import synth
        pb = per_bytes
        in2 = ("layernorm_bwd", pb["layernorm_bwd_input"], lib.ls_layernorm_bwd_input,
               (P["dx2"], P["grad_y2"], P["ffn_out"], P["gamma2"], P["mean2"], P["rstd2"], T, H, P["ws2"], ws, S))
        in1 = ("layernorm_bwd", pb["layernorm_bwd_input"], lib.ls_layernorm_bwd_input,
               (P["dx1"], P["grad_y1"], P["attn_out"], P["gamma1"], P["mean1"], P["rstd1"], T, H, P["ws1"], ws, S))
        if batched_params:
            import ctypes
            vp, i64, sz = ctypes.c_void_p * 2, ctypes.c_int64 * 2, ctypes.c_size_t * 2
            # host arrays of the two jobs, kept alive with the set
            self.jobs = (vp(P["dg2"], P["dg1"]), vp(P["db2"], P["db1"]), i64(T, T), i64(H, H),
                         vp(P["ws2"], P["ws1"]), sz(ws, ws))
            bwd = [in2, in1, ("layernorm_bwd_params", 2 * pb["layernorm_bwd_params"],
                              lib.ls_layernorm_bwd_params_batched, (2, *self.jobs, S), "side")]
        else:
            bwd = [in2, ("layernorm_bwd_params", pb["layernorm_bwd_params"], lib.ls_layernorm_bwd_params,
                         (P["dg2"], P["db2"], T, H, P["ws2"], ws, S), "side"),
                   in1, ("layernorm_bwd_params", pb["layernorm_bwd_params"], lib.ls_layernorm_bwd_params,
                         (P["dg1"], P["db1"], T, H, P["ws1"], ws, S), "side")]
        # (name, algorithmic bytes, ctypes function, args)
        if fused:
            sub1 = [("bias_dropout_residual_layernorm", pb["bias_dropout_residual_layernorm"],
                     lib.ls_bias_dropout_residual_layernorm,
                     (P["attn_out"], P["ln1"], P["mean1"], P["rstd1"], P["attn_proj"], P["attn_bias"], P["residual"],
                      P["gamma1"], P["beta1"], T, H, p, seed, synth.SITE_ATTN_OUT, eps, S))]
            sub2 = [("bias_dropout_residual_layernorm", pb["bias_dropout_residual_layernorm"],
                     lib.ls_bias_dropout_residual_layernorm,
                     (P["ffn_out"], P["ln2"], P["mean2"], P["rstd2"], P["ffn_proj"], P["ffn_bias2"], P["ln1"],
                      P["gamma2"], P["beta2"], T, H, p, seed, synth.SITE_FFN_OUT, eps, S))]
        else:
            sub1 = [("bias_dropout_residual", pb["bias_dropout_residual"], lib.ls_bias_dropout_residual,
                     (P["attn_out"], P["attn_proj"], P["attn_bias"], P["residual"], T, H, p, seed,
                      synth.SITE_ATTN_OUT, S)),
                    ("layernorm_fwd", pb["layernorm_fwd"], lib.ls_layernorm_fwd,
                     (P["ln1"], P["mean1"], P["rstd1"], P["attn_out"], P["gamma1"], P["beta1"], T, H, eps, S))]
            sub2 = [("bias_dropout_residual", pb["bias_dropout_residual"], lib.ls_bias_dropout_residual,
                     (P["ffn_out"], P["ffn_proj"], P["ffn_bias2"], P["ln1"], T, H, p, seed, synth.SITE_FFN_OUT, S)),
                    ("layernorm_fwd", pb["layernorm_fwd"], lib.ls_layernorm_fwd,
                     (P["ln2"], P["mean2"], P["rstd2"], P["ffn_out"], P["gamma2"], P["beta2"], T, H, eps, S))]
        self.launches = [
            ("softmax_fwd", pb["softmax_fwd"], lib.ls_softmax_fwd,
             (P["probs"], P["scores"], B, NH, L, L, None, 0, S)),
            *sub1,
            ("bias_relu_dropout", pb["bias_relu_dropout"], lib.ls_bias_relu_dropout,
             (P["ffn_act"], P["ffn_pre"], P["ffn_bias1"], T, F, p, seed, synth.SITE_FFN_ACT, S)),
            *sub2,
            # LayerNorm backward as its two calls: the input gradient, then the
            # parameter gradients (consumed only by the optimizer; tagged so a
            # caller may put them on a side stream).  batched_params: both
            # LayerNorms' parameter gradients in one call after both input calls.
            *bwd,
            ("softmax_bwd", pb["softmax_bwd"], lib.ls_softmax_bwd,
             (P["dscores"], P["probs"], P["grad_probs"], B * NH * L, L, S)),
        ]

    def run(self, check, side=None):
        issue(self.torch, self.launches, check, side)


def op_of(item_name):
    """The operator a launch item belongs to (the LayerNorm backward's
    parameter call is part of layernorm_bwd)."""
    return item_name[:-len("_params")] if item_name.endswith("_params") else item_name


def issue(torch, items, check, side=None):
    """Issues launch items (name, bytes, fn, args[, "side"]) on the current
    stream, the stream argument (the last of args) replaced by the stream
    used.  Items tagged "side" go to the side stream after an event on the
    current one, and the current stream waits for the side stream at the end;
    with side=None they run in order on the current stream."""
    main = torch.cuda.current_stream()
    forked = False
    for it in items:
        name, _, fn, a = it[:4]
        if len(it) > 4 and side is not None:
            side.wait_stream(main)
            with torch.cuda.stream(side):
                check(name, fn(*a[:-1], side.cuda_stream))
            forked = True
        else:
            check(name, fn(*a[:-1], main.cuda_stream))
    if forked:
        main.wait_stream(side)


def capture_items(torch, items, cap_stream, check, side):
    """One HIP graph of the launch items (side-stream items as a branch that
    joins before the graph ends)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap_stream):
        issue(torch, items, check, side)
    return g


def graph_chunks(n_steps, steps_per_graph):
    """(first step, steps) of each graph when n_steps steps run as graphs of
    steps_per_graph consecutive steps; the last graph holds the steps left
    over, so the graphs cover exactly n_steps steps."""
    return [(i, min(steps_per_graph, n_steps - i)) for i in range(0, n_steps, steps_per_graph)]


def sample_every_graphs(n_graphs, steps_per_graph):
    """Every how many timed graphs one is split to time the dominant kernel
    live: about 24 samples or more, and at least one every ~32 steps' worth."""
    return max(1, min(-(-32 // steps_per_graph), n_graphs // 24))


def capture_steps(torch, runs, cap_stream, check, side):
    """One HIP graph of several steps (ChainSets) in turn, each step's
    side-stream items joined before the next step."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap_stream):
        for s in runs:
            issue(torch, s.launches, check, side)
    return g


def replay_us(torch, graphs, reps):
    """Mean microseconds per graph over reps rounds of the graphs in turn."""
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps * len(graphs)):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * len(graphs))


def build_sets(torch, lib, shape, nsets, p, seed, eps, config=3, fused=True, batched_params=True):
    import synth
    per, counts, total = chain_bytes(shape.tokens, shape.hidden, shape.ffn, shape.heads, shape.seq, fused)
    inputs = synth.chain_inputs(shape, config=config)
    sets = [ChainSet(torch, inputs, shape, lib, per, p, seed, eps, fused, batched_params) for _ in range(nsets)]
    return sets, per, counts, total


# ---------------------------------------------------------------------------
# Oracle CPU baseline
# ---------------------------------------------------------------------------

def chain_slice(inp, shape, s0, nseq):
    """Sequences [s0, s0 + nseq) of the C3 chain inputs (parameters whole)."""
    T0, T1 = s0 * shape.seq, (s0 + nseq) * shape.seq
    return {k: (v[s0:s0 + nseq] if v.ndim == 4 else (v[T0:T1] if v.shape[0] == shape.tokens else v))
            for k, v in inp.items()}


def oracle_chain_pass(sl, shape, p, seed, eps, times=None):
    """One pass of the oracle over every step of the chain, on a slice of it.
    times: a dict that collects each operator's seconds (summed over its calls)."""
    import oracle
    bits = 16

    def run(name, fn, *args):
        t0 = time.perf_counter()
        out = fn(*args)
        if times is not None:
            times[name] = times.get(name, 0.0) + time.perf_counter() - t0
        return out
    probs = run("softmax_fwd", oracle.softmax_fwd, sl["scores"])
    a, l1, m1, r1 = run("bias_dropout_residual_layernorm", oracle.bias_dropout_residual_layernorm, sl["attn_proj"],
                        sl["attn_bias"], sl["residual"], sl["gamma1"], sl["beta1"], p, seed, 0, bits, eps)
    run("bias_relu_dropout", oracle.bias_relu_dropout, sl["ffn_pre"], sl["ffn_bias1"], p, seed, 1, bits)
    f, l2, m2, r2 = run("bias_dropout_residual_layernorm", oracle.bias_dropout_residual_layernorm, sl["ffn_proj"],
                        sl["ffn_bias2"], l1, sl["gamma2"], sl["beta2"], p, seed, 2, bits, eps)
    run("layernorm_bwd", oracle.layernorm_bwd, sl["grad_y2"], f, sl["gamma2"], m2, r2)
    run("layernorm_bwd", oracle.layernorm_bwd, sl["grad_y1"], a, sl["gamma1"], m1, r1)
    k = shape.seq
    run("softmax_bwd", oracle.softmax_bwd, probs.reshape(-1, k), sl["grad_probs"].reshape(-1, k))


def cpu_model():
    """The host CPU's model string (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(shape, p, seed, eps, min_seconds=10.0, max_seconds=30.0):
    """The oracle (fp64 NumPy, single thread) over a bounded sample of the chain:
    4 of the 32 sequences (512 tokens) through every step, repeated until at
    least `min_seconds` of CPU work; scaled to GB/s and tokens/s.  Beside it,
    the same oracle sharded by sequences over the host's cores."""
    import synth
    nseq = 4
    T = nseq * shape.seq
    sl = chain_slice(synth.chain_inputs(shape, config=3), shape, 0, nseq)
    passes = 0
    times = {}
    t0 = time.perf_counter()
    while True:
        oracle_chain_pass(sl, shape, p, seed, eps, times)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el + el / passes > max_seconds:
            break
    per, counts, bytes_per_pass = chain_bytes(T, shape.hidden, shape.ffn, shape.heads, shape.seq)
    per_op = {op: {"ms_per_call": round(1e3 * sec / (passes * counts[op]), 3),
                   "GB/s": round(per[op] * counts[op] * passes / sec / 1e9, 4)} for op, sec in times.items()}
    return {
        "value": round(bytes_per_pass * passes / el / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{passes} pass(es) of the full chain over {nseq} of 32 sequences ({T} of {shape.tokens} tokens), "
                  f"{el:.1f} s; NumPy float64, single thread",
        "tokens_per_s": round(T * passes / el, 1),
        "per_operator": per_op,
        "host_cpus_available": len(os.sched_getaffinity(0)),
        "host_cpu_count": os.cpu_count(),
        "cpu_model": cpu_model(),
        "all_cores": cpu_baseline_sharded(shape, seconds=min_seconds / 2),
        "other_configs": cpu_baseline_other(p, seed, eps, seconds=min(2.0, min_seconds / 5)),
    }


def cpu_baseline_other(p, seed, eps, seconds=2.0):
    """The oracle (single thread) on bounded samples of the other configs:
    the Transformer-big chain over 1 of its 32 sequences, the embedding
    forward and backward over the same 256 tokens, and one Adam step over one
    8M-parameter chunk of the 350M workspace; each repeated for `seconds`."""
    import numpy as np

    import oracle
    import synth

    def repeat(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return n, el
    out = {}
    shape = synth.C4
    T, H = shape.seq, shape.hidden
    sl = chain_slice(synth.chain_inputs(shape, config=4), shape, 0, 1)
    n, el = repeat(lambda: oracle_chain_pass(sl, shape, p, seed, eps))
    _, _, b = chain_bytes(T, H, shape.ffn, shape.heads, shape.seq)
    out["transformer_big_chain"] = {"GB/s": round(b * n / el / 1e9, 4), "tokens_per_s": round(T * n / el, 1),
                                    "sample": f"{n} passes over 1 of {shape.batch} sequences ({T} tokens)"}
    e = synth.embedding_inputs()
    ids, dy = e["ids"][:1], e["grad_out"][:T]
    distinct = int(np.unique(ids).size)
    bits = 16                                   # the dropout decision fields, as in oracle_chain_pass
    n, el = repeat(lambda: oracle.embedding_fwd(ids, e["tok_emb"], e["pos_emb"], e["scale"], p, seed,
                                                synth.SITE_EMBEDDING, bits))
    nb = 4 * T + 2 * H * distinct + 2 * H * T + 2 * T * H
    out["embedding_fwd"] = {"GB/s": round(nb * n / el / 1e9, 4), "tokens_per_s": round(T * n / el, 1),
                            "sample": f"{n} passes over {T} tokens ({distinct} distinct ids)"}
    n, el = repeat(lambda: oracle.embedding_bwd(ids, dy, shape.vocab, e["scale"], p, seed, synth.SITE_EMBEDDING,
                                                bits))
    nb = 4 * T + 2 * T * H + 8 * H * distinct
    out["embedding_bwd"] = {"GB/s": round(nb * n / el / 1e9, 4), "tokens_per_s": round(T * n / el, 1),
                            "sample": f"{n} passes over {T} tokens ({distinct} distinct ids)"}
    pc, gc = synth.adam_chunk(0)
    m0, v0 = np.zeros(pc.size, np.float32), np.zeros(pc.size, np.float32)
    hp = synth.ADAM_HYPER
    n, el = repeat(lambda: oracle.adam_workspace_step(pc, gc, m0, v0, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                                      hp["weight_decay"], 1, hp["grad_scale"], hp["decoupled_wd"]))
    out["adam_workspace_step"] = {"GB/s": round(22 * pc.size * n / el / 1e9, 4),
                                  "params_per_s": round(pc.size * n / el, 1),
                                  "sample": f"{n} steps over one {pc.size}-parameter chunk of the 350M workspace"}
    return out


def cpu_baseline_sharded(shape, seconds):
    """The same oracle passes sharded by sequences over every core this process
    may use: one single-threaded worker process per core, each on its own
    sequences; all start together.  Throughput = all tokens over the longest
    worker's time."""
    import subprocess
    n = max(1, min(len(os.sched_getaffinity(0)), shape.tokens // shape.seq))
    per = -(-(shape.tokens // shape.seq) // n)
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    procs = []
    for w in range(n):
        s0 = w * per
        cnt = min(per, shape.tokens // shape.seq - s0)
        if cnt <= 0:
            break
        procs.append((cnt, subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-worker", str(s0), str(cnt),
                                             str(seconds)], stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True,
                                            env=env, cwd=ROOT)))
    try:
        for _, pr in procs:
            if pr.stdout.readline().strip() != "ready":
                raise RuntimeError("oracle worker did not start")
        for _, pr in procs:
            pr.stdin.write("go\n")
            pr.stdin.flush()
        res = [json.loads(pr.stdout.readline()) for _, pr in procs]
    finally:
        for _, pr in procs:
            pr.stdin.close()
            pr.wait(timeout=120)
    longest = max(r["elapsed"] for r in res)
    tokens = sum(cnt * shape.seq * r["passes"] for (cnt, _), r in zip(procs, res))
    nbytes = sum(chain_bytes(cnt * shape.seq, shape.hidden, shape.ffn, shape.heads, shape.seq)[2] * r["passes"]
                 for (cnt, _), r in zip(procs, res))
    return {"value": round(nbytes / longest / 1e9, 4), "unit": "GB/s", "cores": len(procs),
            "tokens_per_s": round(tokens / longest, 1),
            "sample": f"{len(procs)} single-threaded worker processes, {per} sequence(s) each, "
                      f"{min(r['passes'] for r in res)}+ passes each in {longest:.1f} s"}


def cpu_worker(s0, nseq, seconds):
    """One worker of cpu_baseline_sharded: builds its slice, waits for the start
    line on stdin, runs oracle passes for `seconds`, prints the count."""
    import synth
    shape = synth.C3
    sl = chain_slice(synth.chain_inputs(shape, config=3), shape, s0, nseq)
    print("ready", flush=True)
    sys.stdin.readline()
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle_chain_pass(sl, shape, synth.DROPOUT_P, synth.DROPOUT_SEED, synth.LN_EPS)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    print(json.dumps({"passes": passes, "elapsed": el}), flush=True)


# ---------------------------------------------------------------------------
# Extra rows measured outside the chain (embedding at the Transformer-big
# shape, Adam over the 350M-parameter workspace)
# ---------------------------------------------------------------------------

def extra_rows(torch, ops, eager=False):
    """The rows outside the C3 chain, each on rotated buffer sets (cold): the
    elementwise backward pair at the C3 shapes, the C4 embedding forward and
    backward, and Adam over the 350M-parameter workspace.  eager: every call
    a few times, untimed, outside graphs (the profiler's counter runs
    attribute counters per dispatch)."""
    import numpy as np

    import synth
    out = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    seed, p = synth.DROPOUT_SEED, synth.DROPOUT_P
    cap = torch.cuda.Stream()

    def cold(calls, reps=10):
        """Mean time per call of one graph holding one call per rotated set."""
        if eager:
            for c in calls[:3]:
                c()
            torch.cuda.synchronize()
            return float("nan")
        for c in calls:
            c()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for c in calls:
                c()
        g.replay()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * len(calls))

    def row(shape, us, nbytes, **kw):
        return {"shape": shape, "us": round(us, 2), "bytes": nbytes, "GB/s": round(nbytes / us / 1e3, 1), **kw}

    # Elementwise backward, C3 shapes
    T, H, F = synth.C3.tokens, synth.C3.hidden, synth.C3.ffn
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    rnd = lambda *s: torch.randn(*s, device="cuda", generator=gen).half()  # noqa: E731
    calls = []
    for _ in range(24):
        dy, dx, db = rnd(T, H), torch.empty(T, H, dtype=torch.float16, device="cuda"), rnd(H)
        ws = torch.empty(ops.elementwise_bwd_workspace_bytes(T, H), dtype=torch.uint8, device="cuda")
        calls.append(lambda dy=dy, dx=dx, db=db, ws=ws: ops.bias_dropout_residual_bwd(
            dy, p, seed, synth.SITE_FFN_OUT, dx=dx, dbias=db, workspace=ws))
    nb = 4 * T * H + 2 * H
    out["bias_dropout_residual_bwd"] = row(f"[{T},{H}] -> dx, dbias", cold(calls), nb)
    del calls
    fwd_out = ops.bias_relu_dropout(rnd(T, F), rnd(F), p, seed, synth.SITE_FFN_ACT)
    calls = []
    for _ in range(12):
        dy, o, dx, db = rnd(T, F), fwd_out.clone(), torch.empty(T, F, dtype=torch.float16, device="cuda"), rnd(F)
        ws = torch.empty(ops.elementwise_bwd_workspace_bytes(T, F), dtype=torch.uint8, device="cuda")
        calls.append(lambda dy=dy, o=o, dx=dx, db=db, ws=ws: ops.bias_relu_dropout_bwd(
            dy, o, p, dx=dx, dbias=db, workspace=ws))
    nb = 6 * T * F + 2 * F
    out["bias_relu_dropout_bwd"] = row(f"[{T},{F}] -> dx, dbias (from the forward output)", cold(calls), nb)
    del calls, fwd_out
    torch.cuda.empty_cache()

    # The chain's kernels at the Transformer-big shapes, each alone on enough
    # rotated buffer sets (>= 1.2 GB) to miss the Infinity Cache.
    T4_, H4_, F4_ = synth.C4.tokens, synth.C4.hidden, synth.C4.ffn
    B4_, NH4_, L4_ = synth.C4.batch, synth.C4.heads, synth.C4.seq
    per4, _, _ = chain_bytes(T4_, H4_, F4_, NH4_, L4_)
    sets_for = lambda nbytes: max(4, -(-int(1.2e9) // nbytes))  # noqa: E731
    emp = lambda *s, dt=torch.float16: torch.empty(s, dtype=dt, device="cuda")  # noqa: E731
    c4 = {}

    def c4_row(name, calls):
        us = cold(calls)
        c4[name] = {"us": round(us, 2), "bytes": per4[name], "GB/s": round(per4[name] / us / 1e3, 1),
                    "pct_of_peak": round(100 * per4[name] / us / 1e3 / HBM_PEAK_GBPS, 1)}

    R = sets_for(per4["bias_dropout_residual"])
    bs = [(rnd(T4_, H4_), rnd(H4_), rnd(T4_, H4_), emp(T4_, H4_)) for _ in range(R)]
    c4_row("bias_dropout_residual", [lambda s=s: ops.bias_dropout_residual(s[0], s[1], s[2], p, seed, 0, out=s[3])
                                     for s in bs])
    del bs
    R = sets_for(per4["bias_dropout_residual_layernorm"])
    gm, bt = rnd(H4_).abs() + 0.5, rnd(H4_)
    bs = [(rnd(T4_, H4_), rnd(H4_), rnd(T4_, H4_), emp(T4_, H4_), emp(T4_, H4_), emp(T4_, dt=torch.float32),
           emp(T4_, dt=torch.float32)) for _ in range(R)]
    c4_row("bias_dropout_residual_layernorm",
           [lambda s=s: ops.bias_dropout_residual_layernorm(s[0], s[1], s[2], gm, bt, p, seed, 0, synth.LN_EPS,
                                                            z=s[3], y=s[4], mean=s[5], rstd=s[6]) for s in bs])
    del bs
    R = sets_for(per4["bias_relu_dropout"])
    bs = [(rnd(T4_, F4_), rnd(F4_), emp(T4_, F4_)) for _ in range(R)]
    c4_row("bias_relu_dropout", [lambda s=s: ops.bias_relu_dropout(s[0], s[1], p, seed, 1, out=s[2]) for s in bs])
    del bs
    R = sets_for(per4["layernorm_fwd"])
    bs = [(rnd(T4_, H4_), emp(T4_, H4_), emp(T4_, dt=torch.float32), emp(T4_, dt=torch.float32)) for _ in range(R)]
    c4_row("layernorm_fwd", [lambda s=s: ops.layernorm_fwd(s[0], gm, bt, synth.LN_EPS, y=s[1], mean=s[2], rstd=s[3])
                             for s in bs])
    for s in bs:
        ops.layernorm_fwd(s[0], gm, bt, synth.LN_EPS, y=s[1], mean=s[2], rstd=s[3])
    R2 = sets_for(per4["layernorm_bwd"])
    wsn = ops.layernorm_bwd_workspace_bytes(T4_, H4_)
    bb = [(rnd(T4_, H4_), bs[i % len(bs)], emp(T4_, H4_), emp(H4_), emp(H4_), emp(wsn, dt=torch.uint8))
          for i in range(R2)]
    c4_row("layernorm_bwd", [lambda s=s: ops.layernorm_bwd(s[0], s[1][0], gm, s[1][2], s[1][3], dx=s[2], dgamma=s[3],
                                                           dbeta=s[4], workspace=s[5]) for s in bb])
    del bs, bb
    R = sets_for(per4["softmax_bwd"])
    bs = [(rnd(B4_, NH4_, L4_, L4_), emp(B4_, NH4_, L4_, L4_), rnd(B4_, NH4_, L4_, L4_)) for _ in range(R)]
    c4_row("softmax_fwd", [lambda s=s: ops.softmax_fwd(s[0], y=s[1]) for s in bs])
    c4_row("softmax_bwd", [lambda s=s: ops.softmax_bwd(s[1], s[2], dx=s[0]) for s in bs])
    del bs
    torch.cuda.empty_cache()
    out["transformer_big_kernels"] = c4

    # The two parity configs, timed for the record (launch- and cache-bound:
    # no bandwidth target): the tiny chain at 128 x 256 (the fused block, then
    # the LayerNorm backward's input and parameter calls) and the attention
    # softmax at [8, 12, 128, 128] with per-sequence key lengths, plain and
    # causal.  (Left out of the counter runs: their kernels share names with
    # the rows above.)
    if not eager:
        S1 = synth.C1
        T1, H1 = S1.tokens, S1.hidden
        per1, _, _ = chain_bytes(T1, H1, S1.ffn, S1.heads, S1.seq)
        gm1, bt1, b1 = rnd(H1).abs() + 0.5, rnd(H1), rnd(H1)
        ws1n = ops.layernorm_bwd_workspace_bytes(T1, H1)
        sets1 = [{"x": rnd(T1, H1), "r": rnd(T1, H1), "dy": rnd(T1, H1), "z": emp(T1, H1), "y": emp(T1, H1),
                  "dx": emp(T1, H1), "m": emp(T1, dt=torch.float32), "s": emp(T1, dt=torch.float32),
                  "dg": emp(H1), "db": emp(H1), "ws": emp(ws1n, dt=torch.uint8)} for _ in range(64)]
        calls = []
        for t in sets1:
            calls += [lambda t=t: ops.bias_dropout_residual_layernorm(t["x"], b1, t["r"], gm1, bt1, p, seed, 0,
                                                                      synth.LN_EPS, z=t["z"], y=t["y"], mean=t["m"],
                                                                      rstd=t["s"]),
                      lambda t=t: ops.layernorm_bwd_input(t["dy"], t["z"], gm1, t["m"], t["s"], t["ws"], dx=t["dx"]),
                      lambda t=t: ops.layernorm_bwd_params(T1, H1, t["ws"], dgamma=t["dg"], dbeta=t["db"])]
        us = 3 * cold(calls)
        nb = (per1["bias_dropout_residual_layernorm"] + per1["layernorm_bwd_input"] +
              per1["layernorm_bwd_params"])
        out["tiny_chain"] = row(f"[{T1},{H1}]: fused block, LayerNorm backward input and parameter calls", us, nb,
                                calls_per_chain=3, tokens_per_s=round(T1 / (us * 1e-6), 1))
        del sets1, calls
        inp2 = synth.softmax_inputs()
        kl = d(inp2["key_lengths"])
        e2 = int(np.prod(synth.C2_SHAPE))
        sets2 = [(d(inp2["scores"]), emp(*synth.C2_SHAPE), d(inp2["grad_out"]), emp(*synth.C2_SHAPE))
                 for _ in range(16)]
        for causal in (False, True):
            key = "attention_softmax_fwd" + ("_causal" if causal else "")
            out[key] = row(f"{list(synth.C2_SHAPE)}, per-sequence key lengths" + (", causal" if causal else ""),
                           cold([lambda s=s, c=causal: ops.softmax_fwd(s[0], kl, c, y=s[1]) for s in sets2]), 4 * e2)
        out["attention_softmax_bwd"] = row(f"{list(synth.C2_SHAPE)}",
                                           cold([lambda s=s: ops.softmax_bwd(s[1], s[2], dx=s[3]) for s in sets2]),
                                           6 * e2)
        del sets2
        torch.cuda.empty_cache()

    # Bias + Q/K/V head split and its backward, C3 attention shape
    B, L, NH = synth.C3.batch, synth.C3.seq, synth.C3.heads
    H3 = 3 * H
    calls, bcalls = [], []
    for _ in range(24):
        qkv, bias, o = rnd(T, H3), rnd(H3), torch.empty((3, B, NH, L, H // NH), dtype=torch.float16, device="cuda")
        calls.append(lambda qkv=qkv, bias=bias, o=o: ops.bias_qkv_split(qkv, bias, B, L, NH, out=o))
        dq, db = torch.empty(T, H3, dtype=torch.float16, device="cuda"), rnd(H3)
        ws = torch.empty(ops.elementwise_bwd_workspace_bytes(T, H3), dtype=torch.uint8, device="cuda")
        bcalls.append(lambda o=o, dq=dq, db=db, ws=ws: ops.bias_qkv_split_bwd(o, dqkv=dq, dbias=db, workspace=ws))
    shape = f"[{T},{H3}] <-> 3 x [{B},{NH},{L},{H // NH}]"
    out["bias_qkv_split"] = row(shape, cold(calls), 4 * T * H3 + 2 * H3)
    out["bias_qkv_split_bwd"] = row(shape + " + dbias", cold(bcalls), 4 * T * H3 + 2 * H3)
    del calls, bcalls
    torch.cuda.empty_cache()

    # Embedding, C4
    inp = synth.embedding_inputs()
    ids, P = d(inp["ids"]), d(inp["pos_emb"])
    T4, H4 = inp["grad_out"].shape
    V = inp["tok_emb"].shape[0]
    distinct = int(np.unique(inp["ids"]).size)
    s4 = inp["scale"]
    calls = []
    for _ in range(16):
        E, o = d(inp["tok_emb"]), torch.empty((T4, H4), dtype=torch.float16, device="cuda")
        calls.append(lambda E=E, o=o: ops.embedding_fwd(ids, E, P, s4, p, seed, synth.SITE_EMBEDDING, out=o))
    nb = 4 * T4 + 2 * H4 * distinct + 2 * H4 * synth.C4.seq + 2 * T4 * H4
    out["embedding_fwd"] = row(f"ids [{synth.C4.batch},{synth.C4.seq}], E [{V},{H4}]", cold(calls), nb,
                               distinct_ids=distinct)
    del calls
    torch.cuda.empty_cache()
    sets = [(d(inp["grad_out"]), torch.zeros((V, H4), dtype=torch.float32, device="cuda")) for _ in range(12)]
    acc = [lambda dy=dy, dE=dE: ops.embedding_bwd(ids, dy, dE, s4, p, seed, synth.SITE_EMBEDDING, zero_first=False)
           for dy, dE in sets]
    zf = [lambda dy=dy, dE=dE: ops.embedding_bwd(ids, dy, dE, s4, p, seed, synth.SITE_EMBEDDING, zero_first=True)
          for dy, dE in sets]
    nb = 4 * T4 + 2 * T4 * H4 + 8 * H4 * distinct
    out["embedding_bwd"] = row(f"ids [{synth.C4.batch},{synth.C4.seq}] -> dE [{V},{H4}] fp32 (accumulate)",
                               cold(acc), nb, distinct_ids=distinct, with_zero_fill_us=round(cold(zf), 2))
    del sets, acc, zf, ids, P
    torch.cuda.empty_cache()

    # Cross-entropy criterion, C4: logits [8192, 32768] (537 MB per set)
    T4, V4 = synth.C4.tokens, synth.C4.vocab
    x4 = d(synth.criterion_logits(0, T4))
    y4 = d(synth.criterion_targets())
    eps, gs = synth.CRITERION_SMOOTHING, synth.CRITERION_LOSS_SCALE / T4
    sets = [(x4 if i == 0 else x4.clone(), torch.empty(T4, device="cuda"), torch.empty(T4, device="cuda"),
             torch.empty_like(x4)) for i in range(2)]
    fw = [lambda s=s: ops.cross_entropy_fwd(s[0], y4, eps, -1, loss=s[1], lse=s[2]) for s in sets]
    bw = [lambda s=s: ops.cross_entropy_bwd(s[0], y4, s[2], eps, -1, gs, dlogits=s[3]) for s in sets]
    shape = f"logits [{T4},{V4}], targets Zipf(1.1), smoothing {eps}"
    out["cross_entropy_fwd"] = row(shape, cold(fw), 2 * T4 * V4 + 4 * T4 + 8 * T4)
    out["cross_entropy_bwd"] = row(shape, cold(bw), 4 * T4 * V4 + 4 * T4 + 4 * T4)
    del sets, fw, bw, x4, y4
    torch.cuda.empty_cache()

    # HARS beam top-k, one Transformer-big decoder step: 128 sentences x beam 4 x vocab 32768
    nb_, nk_ = 128, 4
    sets = []
    for _ in range(16):
        lg = torch.randn((nb_, nk_, V4), device="cuda", generator=gen)
        sets.append((torch.log_softmax(lg, dim=-1), torch.randn((nb_, nk_), device="cuda", generator=gen),
                     torch.empty((nb_, nk_), device="cuda"), torch.empty((nb_, nk_), dtype=torch.int32, device="cuda")))
        del lg
    calls = [lambda s=s: ops.beam_topk(s[0], nk_, s[1], top_scores=s[2], top_ids=s[3]) for s in sets]
    out["beam_topk"] = row(f"log-probs [{nb_},{nk_},{V4}] fp32 + beam scores, k {nk_}", cold(calls),
                           4 * nb_ * nk_ * V4 + 4 * nb_ * nk_ + 8 * nb_ * nk_)
    del sets, calls
    torch.cuda.empty_cache()

    # Adam, 350M parameters (7.7 GB per step: larger than every cache by itself)
    n = synth.C5_PARAMS
    gen.manual_seed(5)
    prm = (torch.randn(n, device="cuda", generator=gen) * 0.02).half()
    grd = (torch.randn(n, device="cuda", generator=gen) * 1e-3).half()
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    hp = synth.ADAM_HYPER
    step = [0]

    def adam():
        step[0] += 1
        ops.adam_workspace_step(prm, grd, m, v, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                hp["weight_decay"], step[0], hp["grad_scale"], hp["decoupled_wd"])
    adam()
    torch.cuda.synchronize()
    iters = 2 if eager else 20
    a, b = ev(), ev()
    a.record()
    for _ in range(iters):
        adam()
    b.record()
    torch.cuda.synchronize()
    us_a = a.elapsed_time(b) / iters * 1e3
    out["adam_workspace_step"] = row("350M params, fp16 p/g, fp32 m/v, 1 launch", us_a, 22 * n,
                                     params_per_s=round(n / us_a * 1e6, 1))

    # One GPU's share when the workspace is sharded 8 ways by range (43.75M
    # parameters): the 8 ranges in turn, so no call finds its range in the caches.
    n8 = n // 8
    rngs = [slice(i * n8, (i + 1) * n8) for i in range(8)]

    def adam_range(i):
        r = rngs[i % 8]
        ops.adam_workspace_step(prm[r], grd[r], m[r], v[r], hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                hp["weight_decay"], step[0], hp["grad_scale"], hp["decoupled_wd"])
    for i in range(8):
        adam_range(i)
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record()
    for i in range(0 if eager else 5 * 8):
        adam_range(i)
    b.record()
    torch.cuda.synchronize()
    us_s = float("nan") if eager else a.elapsed_time(b) / 40 * 1e3
    out["adam_workspace_shard"] = row(f"{n8 / 1e6:.2f}M params (350M sharded 8 ways by range), 1 launch", us_s,
                                      22 * n8, params_per_s=round(n8 / us_s * 1e6, 1))

    # The ten steps of the Adam workload from zero moments, and after each
    # the share of fp16 parameters the step left bit-identical: with no fp32
    # master copy an update below half an fp16 spacing of the parameter is
    # lost, which is the trainer's cost in accuracy.
    gen.manual_seed(5)
    prm.copy_((torch.randn(n, device="cuda", generator=gen) * 0.02).half())
    m.zero_()
    v.zero_()
    prev = prm.clone()
    unchanged = []
    for st in range(1, 1 if eager else synth.ADAM_STEPS + 1):
        ops.adam_workspace_step(prm, grd, m, v, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                hp["weight_decay"], st, hp["grad_scale"], hp["decoupled_wd"])
        unchanged.append(round((prm == prev).sum().item() / n, 7))
        prev.copy_(prm)
    out["adam_workspace_step"]["unchanged_fraction_per_step"] = unchanged
    del prev
    del prm, grd, m, v
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# rocprofv3 counter summary -> profiles/
# ---------------------------------------------------------------------------

def is_library_kernel(name):
    """Kernels of this library in a rocprofv3 table: templates appear mangled,
    the others demangled."""
    return name.startswith("_ZN2ls") or name.startswith("ls::")


def calibration_kib(rows):
    """The counter value of the 1 GiB calibration copy: the run's first device
    copy (bench.py makes it before anything else)."""
    copies = sorted((r for r in rows if "copyBuffer" in r["Kernel_Name"]), key=lambda r: int(r["Dispatch_Id"]))
    return float(copies[0]["Counter_Value"]) if copies else None


def summarize_counters(fetch_csv, write_csv):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the dominant kernel, scaled by
    what the same counters read for torch's 1 GiB device copy (a plain copy
    kernel of known size), written to profiles/ with the source hash."""
    import csv

    def read(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r.get("Counter_Name") == counter]
        return rows

    def per_kernel(rows, pred):
        vals = [float(r["Counter_Value"]) for r in rows if pred(r["Kernel_Name"])]
        return sum(vals) / len(vals) if vals else None, len(vals)

    is_dom = lambda k: KERNEL_SYMBOL in k                                    # noqa: E731
    f_rows, w_rows = read(fetch_csv, "FETCH_SIZE"), read(write_csv, "WRITE_SIZE")
    f_dom, nf = per_kernel(f_rows, is_dom)
    w_dom, nw = per_kernel(w_rows, is_dom)
    copy_bytes = 1 << 30
    f_copy, w_copy = calibration_kib(f_rows), calibration_kib(w_rows)
    f_scale = copy_bytes / (f_copy * 1024) if f_copy else None
    w_scale = copy_bytes / (w_copy * 1024) if w_copy else None
    res = {
        "kernel": DOMINANT + " row kernel " + DOMINANT_SHAPE,
        "source_hash": source_hash(),
        "dispatches": [nf, nw],
        "fetch_kib_per_dispatch": f_dom, "write_kib_per_dispatch": w_dom,
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib": f_copy, "write_kib": w_copy,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "traffic_bytes": (f_dom * 1024 * f_scale + w_dom * 1024 * w_scale) if (f_dom and f_scale and w_scale) else None,
    }
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    with open(COUNTERS_FILE, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))
    if f_scale and w_scale:
        write_chain_traffic(f_rows, w_rows, f_scale, w_scale, per_kernel)


# Kernel symbols of each chain operator (regular expressions over the mangled
# names; the LayerNorm forward's last template argument is the fused flag).
CHAIN_SYMBOLS = (
    ("softmax_fwd", ("softmax_fwd_kernel",)),
    ("bias_dropout_residual_layernorm", (r"ln_fwd_kernel\w*Lb1EE",)),
    ("bias_dropout_residual", ("elementwise_vec_kernelILb1ELb0ELb1E",)),       # RESID=1, RELU=0, DROP=1
    ("layernorm_fwd", (r"ln_fwd_kernel\w*Lb0EE",)),
    ("bias_relu_dropout", ("elementwise_vec_kernelILb0ELb1ELb1E",)),
    ("layernorm_bwd", ("ln_bwd_kernel", "ln_bwd_finalize_kernel")),
    ("softmax_bwd", ("softmax_bwd_kernel",)),
)


def write_chain_traffic(f_rows, w_rows, f_scale, w_scale, per_kernel):
    """Measured HBM bytes per launch of every C3 chain kernel (FETCH_SIZE and
    WRITE_SIZE, scaled like the dominant kernel's) against the algorithmic bytes."""
    per, _, _ = chain_bytes(4096, 768, 3072, 12, 128)
    out = ["# HBM traffic per launch: BERT-base layer non-GEMM chain (4096 tokens, hidden 768, FFN 3072)", "",
           "Two `rocprofv3 --pmc` passes of `bench.py --eager` (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), "
           f"scaled by what the same counters read for torch's 1 GiB device copy in the same runs (FETCH x{f_scale:.3f}, "
           f"WRITE x{w_scale:.3f}). Commands, from the repository root on the MI355X machine (R = repository root, "
           "OUT = an output folder):", "", "```",
           "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 240 rocprofv3 --pmc FETCH_SIZE -d $OUT/prof_fetch "
           "-o fetch --output-format csv -- python3 $R/bench.py --eager --steps 12 --warmup 2 --no-cpu --no-extra --no-info",
           "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 240 rocprofv3 --pmc WRITE_SIZE -d $OUT/prof_write "
           "-o write --output-format csv -- python3 $R/bench.py --eager --steps 12 --warmup 2 --no-cpu --no-extra --no-info",
           "python bench.py --summarize-counters $OUT/prof_fetch/fetch_counter_collection.csv "
           "$OUT/prof_write/write_counter_collection.csv", "```", "",
           "Per dispatch for each kernel; per call for each operator (a kernel that one dispatch runs for "
           "several calls, like the batched LayerNorm parameter-gradient finalisation, is counted in proportion "
           "to its dispatches per call of the operator's first kernel).", "",
           "| operator | kernel | dispatches | read MB | written MB | measured MB | algorithmic MB | measured / algorithmic |",
           "|---|---|---|---|---|---|---|---|"]
    for op, syms in CHAIN_SYMBOLS:
        tot, seen, calls = 0.0, False, None
        for sym in syms:
            f, nf = per_kernel(f_rows, lambda k, s=sym: re.search(s, k) is not None)
            w, _ = per_kernel(w_rows, lambda k, s=sym: re.search(s, k) is not None)
            if f is None or w is None:
                continue
            rd, wr = f * 1024 * f_scale / 1e6, w * 1024 * w_scale / 1e6
            calls = nf if calls is None else calls
            tot += (rd + wr) * nf / calls
            seen = True
            out.append(f"| {op} | `{sym}` | {nf} | {rd:.2f} | {wr:.2f} | {rd + wr:.2f} | | |")
        if seen:
            out.append(f"| **{op}** | all | | | | **{tot:.2f}** | {per[op] / 1e6:.2f} | **{tot * 1e6 / per[op]:.3f}** |")
    path = os.path.join(ROOT, "profiles", "chain_bert_base_4096tok_traffic.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("wrote", path)


def other_rows_bytes():
    """Algorithmic bytes per call of every row outside the chain, at the shapes
    extra_rows runs them (the same formulas)."""
    import numpy as np

    import synth
    T, H, F = synth.C3.tokens, synth.C3.hidden, synth.C3.ffn
    H3 = 3 * H
    T4, H4, V4, L4 = synth.C4.tokens, synth.C4.hidden, synth.C4.vocab, synth.C4.seq
    distinct = int(np.unique(synth.embedding_inputs()["ids"]).size)
    per4, _, _ = chain_bytes(T4, H4, synth.C4.ffn, synth.C4.heads, L4)
    nb_, nk_ = 128, 4
    n = synth.C5_PARAMS
    out = {
        "bias_dropout_residual_bwd [4096,768]": 4 * T * H + 2 * H,
        "bias_relu_dropout_bwd [4096,3072]": 6 * T * F + 2 * F,
        "bias_qkv_split [4096,2304]": 4 * T * H3 + 2 * H3,
        "bias_qkv_split_bwd [4096,2304]": 4 * T * H3 + 2 * H3,
        "embedding_fwd C4": 4 * T4 + 2 * H4 * distinct + 2 * H4 * L4 + 2 * T4 * H4,
        "embedding_bwd C4": 4 * T4 + 2 * T4 * H4 + 8 * H4 * distinct,
        "embedding_bwd zero fill C4": 4 * V4 * H4,
        "cross_entropy_fwd C4": 2 * T4 * V4 + 4 * T4 + 8 * T4,
        "cross_entropy_bwd C4": 4 * T4 * V4 + 4 * T4 + 4 * T4,
        "beam_topk 128x4x32768": 4 * nb_ * nk_ * V4 + 4 * nb_ * nk_ + 8 * nb_ * nk_,
        "adam_workspace_step 350M": 22 * n,
        "adam_workspace_shard 43.75M": 22 * (n // 8),
    }
    for k in ("bias_dropout_residual", "bias_dropout_residual_layernorm", "bias_relu_dropout", "layernorm_fwd",
              "layernorm_bwd", "softmax_fwd", "softmax_bwd"):
        out[f"{k} C4"] = per4[k]
    S1 = synth.C1
    per1, _, _ = chain_bytes(S1.tokens, S1.hidden, S1.ffn, S1.heads, S1.seq)
    out["tiny_chain C1 (3 calls)"] = (per1["bias_dropout_residual_layernorm"] + per1["layernorm_bwd_input"] +
                                      per1["layernorm_bwd_params"])
    e2 = int(np.prod(synth.C2_SHAPE))
    out["attention_softmax_fwd C2"] = 4 * e2
    out["attention_softmax_bwd C2"] = 6 * e2
    return out


# Each row outside the chain: (row, kernel-name pattern, grid-size choice, follower).  "largest" /
# "smallest" pick the dispatches of that pattern with the largest / smallest grid (the same kernel
# at two shapes); a follower pattern (a column finalisation) is attributed to the row whose kernel
# is the nearest library dispatch before it.
ROW_KERNELS = (
    ("bias_dropout_residual_bwd [4096,768]", r"ew_bwd_vec_kernelILb0E", None, "colsum_finalize_kernel"),
    ("bias_relu_dropout_bwd [4096,3072]", r"ew_bwd_vec_kernelILb1E", None, "colsum_finalize_kernel"),
    ("bias_dropout_residual C4", r"elementwise_vec_kernelILb1ELb0ELb1E", None, None),
    ("bias_dropout_residual_layernorm C4", r"ln_fwd_kernel\w*Lb1EE", None, None),
    ("bias_relu_dropout C4", r"elementwise_vec_kernelILb0ELb1ELb1E", "largest", None),
    ("layernorm_fwd C4", r"ln_fwd_kernel\w*Lb0EE", None, None),
    ("layernorm_bwd C4", r"ln_bwd_kernel", None, "ln_bwd_finalize_kernel"),
    ("softmax_fwd C4", r"softmax_fwd_kernel", None, None),
    ("softmax_bwd C4", r"softmax_bwd_kernel", None, None),
    ("bias_qkv_split [4096,2304]", r"qkv_split_vec_kernel", None, None),
    ("bias_qkv_split_bwd [4096,2304]", r"qkv_split_bwd_vec_kernel", None, "colsum_finalize_kernel"),
    ("embedding_fwd C4", r"emb_fwd_vec_kernel", None, None),
    ("embedding_bwd C4", r"emb_bwd_sorted_kernel", None, None),
    ("embedding_bwd zero fill C4", r"fill_zero_kernel", None, None),
    ("cross_entropy_fwd C4", r"xent_fwd_vec_kernel", None, None),
    ("cross_entropy_bwd C4", r"xent_bwd_vec_kernel", None, None),
    ("beam_topk 128x4x32768", r"beam_row_topk_kernel", None, "beam_merge_kernel"),
    ("adam_workspace_step 350M", r"adam_kernel", "largest", None),
    ("adam_workspace_shard 43.75M", r"adam_kernel", "smallest", None),
)


def summarize_rows(fetch_csv, write_csv):
    """HBM bytes per call of every row outside the chain, from FETCH_SIZE and
    WRITE_SIZE passes of `bench.py --rows-only --eager`, scaled like the
    chain's counters (by torch's 1 GiB device copy in the same run), against
    the algorithmic bytes; written to profiles/other_rows_traffic.md."""
    import csv
    copy_bytes = 1 << 30

    def load(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r.get("Counter_Name") == counter]
        calib = calibration_kib(rows)
        lib = sorted((r for r in rows if is_library_kernel(r["Kernel_Name"])), key=lambda r: int(r["Dispatch_Id"]))
        return lib, copy_bytes / (calib * 1024)

    f_rows, f_scale = load(fetch_csv, "FETCH_SIZE")
    w_rows, w_scale = load(write_csv, "WRITE_SIZE")

    def per_row(lib, scale):
        """row -> (bytes per dispatch of its kernel, of its follower, dispatch counts)."""
        owner_of = {}                   # dispatch index -> row, for the kernels of every row
        res = {}
        for row, pat, pick, follow in ROW_KERNELS:
            hits = [i for i, r in enumerate(lib) if re.search(pat, r["Kernel_Name"])]
            if pick and hits:
                grids = [int(lib[i]["Grid_Size"]) for i in hits]
                want = max(grids) if pick == "largest" else min(grids)
                hits = [i for i, g in zip(hits, grids) if g == want]
            for i in hits:
                owner_of[i] = row
            main = [float(lib[i]["Counter_Value"]) * 1024 * scale for i in hits]
            res[row] = [main, [], follow]
        for i, r in enumerate(lib):
            for row, (main, fol, follow) in res.items():
                if follow and re.search(follow, r["Kernel_Name"]):
                    j = i - 1
                    while j >= 0 and j not in owner_of:
                        j -= 1
                    if j >= 0 and owner_of[j] == row:
                        fol.append(float(r["Counter_Value"]) * 1024 * scale)
        return res

    fr, wr = per_row(f_rows, f_scale), per_row(w_rows, w_scale)
    alg = other_rows_bytes()
    mean = lambda v: sum(v) / len(v) if v else 0.0  # noqa: E731
    out = ["# HBM traffic per call: the rows outside the BERT-base chain", "",
           "Two `rocprofv3 --pmc` passes of `bench.py --rows-only --eager` (FETCH_SIZE, then WRITE_SIZE, KiB per "
           f"dispatch), scaled by what the same counters read for torch's 1 GiB device copy in the same runs (FETCH "
           f"x{f_scale:.3f}, WRITE x{w_scale:.3f}). A row's bytes are its kernel's mean per dispatch plus, where it "
           "has one, the mean of its second kernel (a column finalisation or merge). Commands, from the repository "
           "root on the MI355X machine (R = repository root, OUT = an output folder):", "", "```",
           "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE -d $OUT/rows_fetch -o fetch "
           "--output-format csv -- python3 $R/bench.py --rows-only --eager",
           "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE -d $OUT/rows_write -o write "
           "--output-format csv -- python3 $R/bench.py --rows-only --eager",
           "python bench.py --summarize-rows $OUT/rows_fetch/fetch_counter_collection.csv "
           "$OUT/rows_write/write_counter_collection.csv", "```", "",
           "| row | dispatches | read MB | written MB | measured MB | algorithmic MB | measured / algorithmic |",
           "|---|---|---|---|---|---|---|"]
    for row, _, _, _ in ROW_KERNELS:
        fm, ff, _ = fr[row]
        wm, wf, _ = wr[row]
        if not fm or not wm:
            out.append(f"| {row} | 0 | | | | {alg[row] / 1e6:.2f} | |")
            continue
        rd, wt = mean(fm) + mean(ff), mean(wm) + mean(wf)
        n = f"{len(fm)}" + (f" + {len(ff)}" if ff else "")
        out.append(f"| {row} | {n} | {rd / 1e6:.2f} | {wt / 1e6:.2f} | {(rd + wt) / 1e6:.2f} | {alg[row] / 1e6:.2f} | "
                   f"{(rd + wt) / alg[row]:.3f} |")
    path = os.path.join(ROOT, "profiles", "other_rows_traffic.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def summarize_trace(trace_csv, out_name, title, note, command, step_kernel=None):
    """Per-kernel duration statistics of the library's kernels from a
    rocprofv3 kernel trace (one row per kernel and grid size), written to
    profiles/<out_name> with the command that made the trace.  step_kernel: a
    kernel-name fragment that runs once per step; then the sum of kernel
    durations per step is given too."""
    import csv
    import statistics
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        name = r["Kernel_Name"]
        if not is_library_kernel(name):
            continue
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        grid = int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1)
        wg = int(r["Workgroup_Size_X"]) * int(r.get("Workgroup_Size_Y") or 1) * int(r.get("Workgroup_Size_Z") or 1)
        groups.setdefault((name, grid // max(1, wg)), []).append(d)
    total = sum(sum(v) for v in groups.values())
    rows = []
    for (name, blocks), v in groups.items():
        v = sorted(v)
        q = lambda f: v[min(len(v) - 1, int(f * len(v)))]  # noqa: E731
        short = name if len(name) <= 110 else name[:107] + "..."
        rows.append((sum(v), f"| `{short}` | {blocks} | {len(v)} | {statistics.fmean(v):.2f} | {q(0.1):.2f} | "
                             f"{statistics.median(v):.2f} | {q(0.9):.2f} | {v[0]:.2f} | {v[-1]:.2f} | "
                             f"{100 * sum(v) / total:.1f} |"))
    rows.sort(reverse=True)
    if step_kernel:
        steps = sum(len(v) for (name, _), v in groups.items() if step_kernel in name)
        if steps:
            note += (f"\n\nSum of the library's kernel durations per step: {total / steps:.2f} us ({steps} steps "
                     f"traced; the step's own wall time, dispatch gaps included, is the bench line's ms_per_step).")
    out = [f"# rocprofv3 kernel statistics: {title}", "", note, "",
           "Command (from the repository root on the MI355X machine; R = repository root, OUT = an output folder):",
           "", "```", command, "```", "",
           "Durations per dispatch from the kernel trace (microseconds); one row per kernel and grid size.", "",
           "| kernel | blocks | calls | avg us | p10 us | median us | p90 us | min us | max us | % of library time |",
           "|---|---|---|---|---|---|---|---|---|---|"] + [r for _, r in rows]
    path = os.path.join(ROOT, "profiles", out_name)
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("wrote", path)


def stored_traffic():
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_hash") != source_hash():
        return None
    return c.get("traffic_bytes")


# ---------------------------------------------------------------------------

def transformer_big_chain(torch, lib, check, cap_stream, side, p, seed, eps, nsets=3, reps=20):
    """The Transformer-big layer (8192 tokens, hidden 1024, 16 heads, FFN 4096)
    through the same calls as the BERT-base step plus the embedding forward and backward
    (vocabulary 32768, Zipf ids, fp32 gradient accumulated) on 3 rotated
    buffer sets (about 0.9 GB each), all three steps in one HIP graph (and,
    for comparison, one graph per step)."""
    import numpy as np

    import synth
    shape = synth.C4
    sets, per, counts, total = build_sets(torch, lib, shape, nsets, p, seed, eps, config=4)
    inp = synth.embedding_inputs()
    distinct = int(np.unique(inp["ids"]).size)
    T, H, V, L = shape.tokens, shape.hidden, shape.vocab, shape.seq
    emb_f = 4 * T + 2 * H * distinct + 2 * H * L + 2 * T * H
    emb_b = 4 * T + 2 * T * H + 8 * H * distinct
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    ids, P = d(inp["ids"]), d(inp["pos_emb"])
    keep = []
    for s in sets:
        E, dy = d(inp["tok_emb"]), d(inp["grad_out"])
        out = torch.empty((T, H), dtype=torch.float16, device="cuda")
        dE = torch.zeros((V, H), dtype=torch.float32, device="cuda")
        keep.append((E, dy, out, dE))
        S = torch.cuda.current_stream().cuda_stream
        s.launches.append(("embedding_fwd", emb_f, lib.ls_embedding_fwd,
                           (out.data_ptr(), ids.data_ptr(), E.data_ptr(), P.data_ptr(), shape.batch, L, H, V, L,
                            inp["scale"], p, seed, synth.SITE_EMBEDDING, S)))
        s.launches.append(("embedding_bwd", emb_b, lib.ls_embedding_bwd,
                           (dE.data_ptr(), ids.data_ptr(), dy.data_ptr(), shape.batch, L, H, V, inp["scale"], p, seed,
                            synth.SITE_EMBEDDING, 0, S)))
        s.run(check, side)
    torch.cuda.synchronize()
    whole = [capture_steps(torch, sets, cap_stream, check, side)]
    us = replay_us(torch, whole, reps) / nsets
    per_step = [capture_steps(torch, [s], cap_stream, check, side) for s in sets]
    us1 = replay_us(torch, per_step, reps)
    nbytes = total + emb_f + emb_b
    out = {"shape": "8192 tokens (32 x 256), hidden 1024, 16 heads, FFN 4096, vocab 32768",
           "calls_per_step": len(sets[0].launches),
           "kernels_per_step": len(sets[0].launches),
           "us_per_step": round(us, 2), "bytes_per_step": nbytes,
           "GB/s": round(nbytes / us / 1e3, 1), "tokens_per_s": round(T / (us * 1e-6), 1),
           "rotated_sets": nsets, "steps_per_graph": nsets,
           "one_graph_per_step": {"us_per_step": round(us1, 2), "GB/s": round(nbytes / us1 / 1e3, 1),
                                  "tokens_per_s": round(T / (us1 * 1e-6), 1)}}
    del whole, per_step, sets, keep
    torch.cuda.empty_cache()
    return out


def attainable(torch, lib, check, cap_stream, dom_bytes, sizes=None):
    """Bandwidth the device reaches with the operators' access pattern: the
    library's reference copy and read kernels over 1 GiB buffers, and a copy
    moving the dominant kernel's byte count, rotated over enough buffers to
    stay out of the 256 MB Infinity Cache.  sizes ({name: bytes}): a cold
    copy of each kernel's own byte count (half read, half written), the
    reference its time is compared with."""
    def rate(pairs, fn, moved, reps=10):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            st = torch.cuda.current_stream().cuda_stream
            for a, b in pairs:
                check(fn.__name__, fn(a.data_ptr(), b.data_ptr(), b.numel(), st))
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * len(pairs))
        return round(moved / us / 1e3, 1), round(us, 2)

    out = {"kernels": "ls_probe_copy / ls_probe_read (16-byte non-temporal accesses, 256-thread blocks)"}
    big = 1 << 30
    pairs = [(torch.empty(big, dtype=torch.uint8, device="cuda"), torch.ones(big, dtype=torch.uint8, device="cuda"))
             for _ in range(2)]
    out["copy_1GiB_GBps"], _ = rate(pairs, lib.ls_probe_copy, 2 * big)
    sinks = [(torch.empty(big // 1024, dtype=torch.float32, device="cuda"), b) for _, b in pairs]
    out["read_1GiB_GBps"], _ = rate(sinks, lib.ls_probe_read, big + big // 256)
    del pairs, sinks
    half = (dom_bytes // 2) // 16 * 16
    pairs = [(torch.empty(half, dtype=torch.uint8, device="cuda"), torch.ones(half, dtype=torch.uint8, device="cuda"))
             for _ in range(24)]
    out["copy_dominant_bytes_GBps"], out["copy_dominant_bytes_us"] = rate(pairs, lib.ls_probe_copy, 2 * half)
    out["copy_dominant_bytes"] = 2 * half
    del pairs
    torch.cuda.empty_cache()
    if sizes:
        measured, table = {}, {}
        for name, nbytes in sizes.items():
            half = (nbytes // 2) // 16 * 16
            if half not in measured:
                n_pairs = max(2, -(-int(1.5e9) // (2 * half)))
                pairs = [(torch.empty(half, dtype=torch.uint8, device="cuda"),
                          torch.ones(half, dtype=torch.uint8, device="cuda")) for _ in range(n_pairs)]
                measured[half] = rate(pairs, lib.ls_probe_copy, 2 * half)[1]
                del pairs
                torch.cuda.empty_cache()
            table[name] = {"bytes": nbytes, "copy_us": measured[half]}
        out["same_size_copy"] = table
    return out


def step_variants(torch, lib, check, cap_stream, p, seed, eps, nsets=12, graph_steps=12, reps=20):
    """The same BERT-base step in other forms, each on its own rotated sets
    and, like the timed steps, in HIP graphs of graph_steps steps: the
    measured step in one graph per step; bias+dropout+residual and LayerNorm
    as two operators each and each LayerNorm's parameter gradients in a call
    of their own (unfused); the fused step with each LayerNorm's parameter
    gradients in a call of their own; and the fused step with the batched
    parameter gradients on a side stream (a branch of the graph, joined at
    the end of each step)."""
    import synth
    shape = synth.C3
    out = {}
    side = torch.cuda.Stream()         # default priority, like every stream here
    for key, fused, batched, side_, g_steps in (
            ("one_graph_per_step", True, True, None, 1),
            ("unfused", False, False, None, graph_steps),
            ("fused_parameter_gradients_per_layernorm", True, False, None, graph_steps),
            ("fused_parameter_gradients_on_side_stream", True, True, side, graph_steps)):
        sets, per, counts, total = build_sets(torch, lib, shape, nsets, p, seed, eps, fused=fused,
                                              batched_params=batched)
        for s in sets:
            s.run(check, side_)
        graphs = [capture_steps(torch, sets[i:i + g_steps], cap_stream, check, side_)
                  for i in range(0, nsets, g_steps)]
        us = replay_us(torch, graphs, reps) / g_steps
        out[key] = {"calls_per_step": len(sets[0].launches), "steps_per_graph": g_steps, "us_per_step": round(us, 2),
                    "bytes_per_step": total, "GB/s": round(total / us / 1e3, 1),
                    "tokens_per_s": round(shape.tokens / (us * 1e-6), 1)}
        del graphs, sets
        torch.cuda.empty_cache()
    return out


def warm_chain_us(torch, s, cap_stream, check, side, graph_steps=1, reps=100):
    """One buffer set stepped again and again (graph_steps steps per graph):
    the chain with its tensors cache-resident."""
    g = capture_steps(torch, [s] * graph_steps, cap_stream, check, side)
    return replay_us(torch, [g], reps) / graph_steps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=12, help="rotated buffer sets (cold-cache measurement)")
    ap.add_argument("--graph-steps", type=int, default=0,
                    help="steps per HIP graph in the timed region (a divisor of --sets; default: --sets)")
    ap.add_argument("--sample-every", type=int, default=0,
                    help="every Nth timed graph runs the dominant kernel between its own events "
                         "(default: about 20-30 samples over the timed region)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the embedding / Adam rows")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel directly instead of replaying HIP graphs (profiler runs)")
    ap.add_argument("--no-info", action="store_true", help="skip the per-kernel and warm-chain information")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--rows-only", action="store_true",
                    help="only the rows outside the chain (with --eager: untimed, for counter runs)")
    ap.add_argument("--summarize-rows", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-trace", nargs=2, metavar=("chain|rows", "KERNEL_TRACE_CSV"))
    ap.add_argument("--cpu-worker", nargs=3, metavar=("SEQ0", "NSEQ", "SECONDS"), help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_worker:
        cpu_worker(int(args.cpu_worker[0]), int(args.cpu_worker[1]), float(args.cpu_worker[2]))
        return 0
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return 0
    if args.summarize_rows:
        summarize_rows(*args.summarize_rows)
        return 0
    if args.summarize_trace:
        which, path = args.summarize_trace
        if which == "chain":
            summarize_trace(path, "chain_bert_base_4096tok_kernel_stats.md",
                            "BERT-base layer non-GEMM step (4096 tokens, hidden 768, FFN 3072), 12 rotated buffer sets",
                            "Under the kernel trace every dispatch waits for the profiler, so each kernel starts on an "
                            "idle GPU and its end includes the profiler's completion handling: durations are longer "
                            "than in the untraced step (compare p10 with the live figures in the bench line).",
                            "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d $OUT/prof_trace -o trace "
                            "--output-format csv -- python3 $R/bench.py --steps 200 --warmup 20 --no-cpu --no-extra "
                            "--no-info\npython $R/bench.py --summarize-trace chain $OUT/prof_trace/trace_kernel_trace.csv",
                            step_kernel="ln_bwd_finalize_kernel")
        else:
            summarize_trace(path, "other_rows_kernel_stats.md", "rows outside the chain",
                            "Elementwise backwards and bias + Q/K/V split at the BERT-base shapes; the chain's kernels "
                            "at the Transformer-big shapes; embedding, cross-entropy (8192 tokens, vocabulary 32768) "
                            "and HARS top-k (128 x 4 x 32768); Adam over 350M parameters and one 8-way shard of it. "
                            "Each row on rotated buffer sets, as in bench.py's other_rows.",
                            "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d $OUT/rows_trace -o rows "
                            "--output-format csv -- python3 $R/bench.py --rows-only\npython $R/bench.py "
                            "--summarize-trace rows $OUT/rows_trace/rows_kernel_trace.csv")
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the operators "
              "shard by token rows with no exchange, and that multi-GPU leg is not built", file=sys.stderr)
        return 2

    import torch

    import synth
    from non_gemm_amd import _lib, ops
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    lib = _lib.load()
    shape = synth.C3
    p, seed, eps = synth.DROPOUT_P, synth.DROPOUT_SEED, synth.LN_EPS

    def check(name, rc):
        if rc != 0:
            _lib.check(name, rc)

    # Calibration copy of known size (read by the rocprofv3 counter runs).
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if args.rows_only:
        print(json.dumps({"other_rows": extra_rows(torch, ops, eager=args.eager)}), flush=True)
        return 0

    sets, per, counts, total = build_sets(torch, lib, shape, args.sets, p, seed, eps)
    footprint = sum(sum(t.numel() * t.element_size() for t in s.t.values()) for s in sets)
    # The step runs on one stream: the LayerNorm parameter gradients in line.
    # (A side-stream branch for them, joined at the end of the step, measured
    # far slower: see step_variants.)
    side = None
    for s in sets:                     # first launches outside any capture
        s.run(check, side)
    torch.cuda.synchronize()

    # The timed steps run as HIP graphs of G consecutive steps each (G =
    # --graph-steps, by default every rotated set in turn: the 12 layers of
    # BERT-base, each on its own buffers, as a whole training iteration would
    # be captured).  A graph's launch costs about 5 us of its own, so one
    # graph per step carries that cost in every step (step_variants reports
    # that form too).  Every SAMPLE-th graph of the timed region runs split
    # around its first step's dominant kernel (graph A, the kernel launched
    # directly between two fence-free events, graph B), so the events sample
    # the kernel live while the other graphs run whole.
    dom_idx = [i for i, l in enumerate(sets[0].launches) if l[0] == DOMINANT][0]
    cap_stream = torch.cuda.Stream()
    n_launch = len(sets[0].launches)
    G = args.graph_steps or len(sets)
    if not 1 <= G <= len(sets) or len(sets) % G:
        print(f"--graph-steps {G} must divide --sets {len(sets)}", file=sys.stderr)
        return 2
    stream = torch.cuda.current_stream()
    S = stream.cuda_stream

    def chunks(n_steps):
        return graph_chunks(n_steps, G)

    graphs = {}                        # (first set, steps) -> (whole, A, B, dominant call)

    def graph_of(i, n):
        key = (i % len(sets), n)
        if key not in graphs:
            run = [sets[(key[0] + k) % len(sets)] for k in range(n)]
            items = [it for s in run for it in s.launches]
            d = run[0].launches[dom_idx]
            graphs[key] = (capture_items(torch, items, cap_stream, check, side),
                           capture_items(torch, items[:dom_idx], cap_stream, check, side),
                           capture_items(torch, items[dom_idx + 1:], cap_stream, check, side),
                           (d[2], d[3][:-1] + (S,)))
        return graphs[key]
    K = args.steps
    for i, n in chunks(args.warmup) + chunks(K):     # every graph captured before the timed region
        graph_of(i, n)
    torch.cuda.synchronize()
    # A sampled graph (two graphs around a direct launch) costs several us
    # more than a whole one, so only every SAMPLE-th graph is split: about
    # 20-30 samples for the kernel's mean, little of that cost in the step.
    n_graphs = len(chunks(K))
    SAMPLE = args.sample_every if args.sample_every > 0 else sample_every_graphs(n_graphs, G)

    def run_graph(c, i, n, ev=None):
        """Steps i .. i+n-1 (graph c of the region); with ev, a sampled one if c % SAMPLE == 0."""
        sampled = ev is not None and c % SAMPLE == 0
        if args.eager:
            for k in range(n):
                s = sets[(i + k) % len(sets)]
                if sampled and k == 0:
                    issue(torch, s.launches[:dom_idx], check, side)
                    ev.arm(c // SAMPLE, lib)
                    fn, a = s.launches[dom_idx][2], s.launches[dom_idx][3][:-1] + (S,)
                    check(DOMINANT, fn(*a))
                    issue(torch, s.launches[dom_idx + 1:], check, side)
                else:
                    issue(torch, s.launches, check, side)
            return
        g_full, g_a, g_b, (fn, a) = graph_of(i, n)
        if not sampled:
            g_full.replay()
            return
        g_a.replay()
        ev.arm(c // SAMPLE, lib)
        check(DOMINANT, fn(*a))
        g_b.replay()

    for c, (i, n) in enumerate(chunks(args.warmup)):
        run_graph(c, i, n)
    torch.cuda.synchronize()

    kev = KernelEvents((n_graphs + SAMPLE - 1) // SAMPLE)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record()
    for c, (i, n) in enumerate(chunks(K)):
        run_graph(c, i, n, kev)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = t_start.elapsed_time(t_end)
    ms_step = gpu_ms / K
    dom_us = kev.mean_us()
    kev.close()
    dom_bytes = per[DOMINANT + "_input"]        # the row kernel's own bytes (dgamma/dbeta come from the params call)
    achieved = dom_bytes / dom_us / 1e3          # GB/s

    # Informational: per-kernel cold times (graphs of R launches of one kind) and
    # the warm (single buffer set) chain.
    kernels = {}
    for name in ([] if args.no_info else counts):
        # the whole operator, its calls in order on one stream
        g = capture_items(torch, [it for s in sets for it in s.launches if op_of(it[0]) == name], cap_stream, check,
                          None)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (reps * len(sets) * counts[name])
        kernels[name] = {"us": round(us, 2), "bytes": per[name], "GB/s": round(per[name] / us / 1e3, 1),
                         "per_step": counts[name]}
    # The Philox rounds' cost: bias+ReLU+dropout (the lowest bytes per
    # decision of the chain) at p = 0, which skips the rounds, against p = 0.1.
    philox = None
    if "bias_relu_dropout" in kernels:
        items = []
        for s in sets:
            for it in s.launches:
                if it[0] == "bias_relu_dropout":
                    a = list(it[3])
                    a[5] = 0.0                                   # p
                    items.append((it[0], it[1], it[2], tuple(a)))
        g0 = capture_items(torch, items, cap_stream, check, None)
        us0 = replay_us(torch, [g0], 20) / len(items)
        us1 = kernels["bias_relu_dropout"]["us"]
        elems = shape.tokens * shape.ffn
        philox = {"kernel": f"bias_relu_dropout [{shape.tokens},{shape.ffn}]", "us_p0.1": us1, "us_p0": round(us0, 2),
                  "extra_us": round(us1 - us0, 2), "extra_ps_per_element": round((us1 - us0) * 1e6 / elems, 4),
                  "share_of_kernel": round((us1 - us0) / us1, 4),
                  # from the generated code: per call of 8 decisions, 20 v_mad_u64_u32 and 20 v_bitop3_b32
                  # (ten rounds, two products and two three-way XORs each), then 8 compares and selects
                  "valu_instructions_per_element": (20 + 20 + 16) / 8}
        del g0
    # The largest single launch, from the same cold graph timing (not live events).
    largest = None
    if LARGEST in kernels:
        k = kernels[LARGEST]
        largest = {"bound": "hbm", "kernel": f"{LARGEST} [4096,3072]", "achieved": k["GB/s"],
                   "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(k["GB/s"] / HBM_PEAK_GBPS, 4),
                   "algorithmic_bytes": per[LARGEST], "avg_duration_us": k["us"],
                   "timing": "cold: a graph of back-to-back launches over the rotated sets, events around it"}
    warm_us = None
    if not args.no_info:
        warm_us = warm_chain_us(torch, sets[0], cap_stream, check, side, G)
    dispatch = {}
    for it in sets[0].launches:
        name, _, fn, args_ = it[:4]
        check(name, fn(*args_))
        dispatch[name] = _lib.last_dispatch()
    torch.cuda.synchronize()
    del graphs, sets
    torch.cuda.empty_cache()
    variants = None if args.no_info else step_variants(torch, lib, check, cap_stream, p, seed, eps,
                                                       nsets=args.sets, graph_steps=G)
    copy_sizes = {**{f"{k} C3": per[k] for k in kernels}, **other_rows_bytes()}
    reach = None if args.no_info else attainable(torch, lib, check, cap_stream, dom_bytes, copy_sizes)
    if reach is not None:
        for k in kernels:
            kernels[k]["pct_of_same_size_copy"] = round(
                100 * reach["same_size_copy"][f"{k} C3"]["copy_us"] / kernels[k]["us"], 1)
    big = None if args.no_info else transformer_big_chain(torch, lib, check, cap_stream, side, p, seed, eps)

    extra = None if args.no_extra else extra_rows(torch, ops)
    cpu = None if args.no_cpu else cpu_baseline(shape, p, seed, eps)

    value = total / (ms_step * 1e-3) / 1e9
    result = {
        "metric": "achieved HBM GB/s (% of peak) + tokens/s for layer non-GEMM chain, BERT-base",
        "value": round(value, 1),
        "unit": "GB/s",
        "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(shape.tokens / (ms_step * 1e-3), 1),
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "bert-base-layer-non-gemm-chain", "tokens": shape.tokens, "batch": shape.batch,
                   "seq_len": shape.seq, "hidden": shape.hidden, "heads": shape.heads, "ffn": shape.ffn,
                   "dropout_p": p, "chain_bytes_per_step": total, "rotated_sets": args.sets,
                   "steps_per_graph": G,
                   "footprint_bytes": footprint, "launches_per_step": n_launch,
                   "kernels_per_step": n_launch,
                   "fused_bias_dropout_residual_layernorm": True},
        "roofline": {"bound": "hbm", "kernel": f"{DOMINANT} row kernel {DOMINANT_SHAPE}",
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": stored_traffic(), "algorithmic_bytes": dom_bytes,
                     "avg_duration_us": round(dom_us, 3),
                     "samples": (n_graphs + SAMPLE - 1) // SAMPLE, "sample_every_graphs": SAMPLE,
                     # the whole operator (row kernel, then its parameter finalisation on the same stream),
                     # from the cold per-operator timing
                     "op_level": None if DOMINANT not in kernels else {
                         "algorithmic_bytes": per[DOMINANT], "us": kernels[DOMINANT]["us"],
                         "achieved": kernels[DOMINANT]["GB/s"],
                         "frac": round(kernels[DOMINANT]["GB/s"] / HBM_PEAK_GBPS, 4)}},
        "roofline_largest_launch": largest,
        "philox_cost": philox,
        "cpu_baseline": cpu,
        "kernels_cold": kernels,
        "warm_chain_us": None if warm_us is None else round(warm_us, 2),
        "attainable_hbm": reach,
        "dispatch": dispatch,
        "step_variants": variants,
        "transformer_big_chain": big,
        "other_rows": extra,
        "wall_s_timed": round(wall, 4),
        "device": torch.cuda.get_device_properties(0).gcnArchName,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
