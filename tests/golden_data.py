"""Reader for the text fixtures under tests/golden/: '#' starts a comment
(each file's comments carry its citation), every other line is
'key = value' with a number or a space-separated list of numbers."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, value = (s.strip() for s in line.split("=", 1))
            nums = [float(v) for v in value.split()]
            out[key] = nums[0] if len(nums) == 1 else np.array(nums)
    return out


def hars_example():
    """(log_probs float32 [1, beam, vocab], k, page's candidate and survivor counts)."""
    d = load("hars_beam2_vocab8.txt")
    beam, vocab = int(d["beam"]), int(d["vocab"])
    lp = np.stack([d[f"logits_beam{i}"] for i in range(beam)]).astype(np.float32).reshape(1, beam, vocab)
    return lp, int(d["k"]), int(d["candidates"]), int(d["survivors"])


def beam_candidates_example():
    """(log_probs float32 [1, beam, vocab], beam_scores float32 [1, beam],
    hand-computed candidates float32 [1, beam, vocab], k, top ids, top scores)."""
    d = load("beam_candidates_fp32.txt")
    beam, vocab = int(d["beam"]), int(d["vocab"])
    lp = np.stack([d[f"log_probs_beam{i}"] for i in range(beam)]).astype(np.float32).reshape(1, beam, vocab)
    bs = np.asarray(d["beam_scores"], np.float32).reshape(1, beam)
    c = np.stack([d[f"candidates_beam{i}"] for i in range(beam)]).astype(np.float32).reshape(1, beam, vocab)
    ids = np.asarray(d["top_ids"]).astype(np.int32).reshape(1, -1)
    scores = np.asarray(d["top_scores"], np.float32).reshape(1, -1)
    return lp, bs, c, int(d["k"]), ids, scores
