"""Seeded synthetic inputs shaped like the pages' workloads.

This module is shared by the tests, ``bench.py`` and the CPU baseline.  It
holds no operator arithmetic: it only draws arrays (NumPy PCG64, sampled in
float64 and rounded once to fp16) and describes the five workloads:

* C1 tiny fused chain: 128 tokens x hidden 256.
* C2 attention softmax: scores [8, 12, 128, 128] ~ N(0, 3), key lengths
  U{16..128} per sequence, causal variant.
* C3 BERT-base layer: 4096 tokens (32 x 128), hidden 768, 12 heads, FFN 3072.
* C4 Transformer-big layer + embedding: 8192 tokens (32 x 256), hidden 1024,
  16 heads, FFN 4096, vocab 32768 with Zipf(1.1) token ids, scale sqrt(1024),
  sinusoidal positions.
* C5 Adam over 350 M fp16 parameters ~ N(0, 0.02), gradients ~ N(0, 1e-3).

N(mu, sigma) below always means standard deviation sigma.  The pages measure on
BERT fine-tuning and on WMT14 En-De Transformer-big training; no dataset or
trained weight is used here, only tensors of those layers' shapes.
"""

from dataclasses import dataclass

import numpy as np

DROPOUT_SEED = 0x0123456789ABCDEF
# One Philox stream word per dropout site of a layer.
SITE_ATTN_OUT = 0      # bias + dropout + residual after the attention projection
SITE_FFN_ACT = 1       # bias + ReLU + dropout after the first FFN GEMM
SITE_FFN_OUT = 2       # bias + dropout + residual after the second FFN GEMM
SITE_EMBEDDING = 3     # embedding dropout


@dataclass(frozen=True)
class LayerShape:
    name: str
    batch: int
    seq: int
    hidden: int
    heads: int
    ffn: int
    vocab: int = 0

    @property
    def tokens(self):
        return self.batch * self.seq


C1 = LayerShape("tiny-chain-128x256", batch=1, seq=128, hidden=256, heads=4, ffn=1024)
C3 = LayerShape("bert-base-layer-4096tok", batch=32, seq=128, hidden=768, heads=12, ffn=3072)
C4 = LayerShape("transformer-big-layer-8192tok", batch=32, seq=256, hidden=1024, heads=16,
                ffn=4096, vocab=32768)
C2_SHAPE = (8, 12, 128, 128)
C5_PARAMS = 350_000_000
C5_CHUNK = 8 * 1024 * 1024
DROPOUT_P = 0.1
LN_EPS = 1e-5


def rng(config, stream=0):
    """Independent PCG64 stream for (config number, sub-stream)."""
    return np.random.default_rng([1000 + int(config), int(stream)])


def normal16(gen, shape, std, mean=0.0):
    return gen.normal(mean, std, size=shape).astype(np.float16)


def uniform16(gen, shape, lo, hi):
    return gen.uniform(lo, hi, size=shape).astype(np.float16)


# Ratios |mean| / std of the offset rows used to probe the one-pass variance.
OFFSET_RATIOS = (0.0, 1.0, 3.0, 10.0, 30.0, 100.0, 1000.0)


def offset_rows16(gen, rows, hidden, ratios=OFFSET_RATIOS, std=1.0):
    """Rows ~ N(m_r, std) with m_r = +-ratio * std, the ratios taken in turn
    and the sign alternating every len(ratios) rows (post-residual
    activations whose mean is large next to their spread)."""
    ratios = np.asarray(ratios, np.float64)
    r = np.arange(rows)
    sign = np.where((r // ratios.size) % 2 == 0, 1.0, -1.0)
    means = sign * ratios[r % ratios.size] * std
    return (means[:, None] + gen.normal(0.0, std, size=(rows, hidden))).astype(np.float16)


def zipf_ids(gen, shape, vocab, s):
    """Token ids from a Zipf law truncated to ranks 1..vocab, P(k) ~ k^-s.

    Sampled by inverting the cumulative distribution; id = rank - 1.
    """
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    w = ranks ** (-float(s))
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = gen.random(size=shape)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def sinusoid_table(max_pos, hidden):
    """Fixed sinusoidal position table, interleaved: even columns sin, odd cos.

    P[pos, 2k] = sin(pos / 10000^(2k/H)), P[pos, 2k+1] = cos(same angle).
    Built in float64 and rounded once to fp16; it is an input, not trained.
    """
    pos = np.arange(max_pos, dtype=np.float64)[:, None]
    k2 = np.arange(0, hidden, 2, dtype=np.float64)[None, :]
    angle = pos / np.power(10000.0, k2 / hidden)
    table = np.empty((max_pos, hidden), dtype=np.float64)
    table[:, 0::2] = np.sin(angle)
    table[:, 1::2] = np.cos(angle[:, : hidden // 2])
    return table.astype(np.float16)


def chain_inputs(shape, config):
    """Activations, parameters and incoming gradients for one layer's chain.

    x, residual, grad_y ~ N(0, 1); biases ~ N(0, 0.02); gamma ~ U(0.5, 1.5);
    beta ~ N(0, 0.1).  Attention scores ~ N(0, 1) (C3/C4 use full rows).
    """
    g = rng(config)
    t, h, f = shape.tokens, shape.hidden, shape.ffn
    a = (shape.batch, shape.heads, shape.seq, shape.seq)
    return {
        "scores": normal16(g, a, 1.0),
        "grad_probs": normal16(g, a, 1.0),
        "attn_proj": normal16(g, (t, h), 1.0),
        "attn_bias": normal16(g, (h,), 0.02),
        "residual": normal16(g, (t, h), 1.0),
        "ffn_pre": normal16(g, (t, f), 1.0),
        "ffn_bias1": normal16(g, (f,), 0.02),
        "ffn_proj": normal16(g, (t, h), 1.0),
        "ffn_bias2": normal16(g, (h,), 0.02),
        "gamma1": uniform16(g, (h,), 0.5, 1.5),
        "beta1": normal16(g, (h,), 0.1),
        "gamma2": uniform16(g, (h,), 0.5, 1.5),
        "beta2": normal16(g, (h,), 0.1),
        "grad_y1": normal16(g, (t, h), 1.0),
        "grad_y2": normal16(g, (t, h), 1.0),
    }


def softmax_inputs(config=2, shape=C2_SHAPE):
    """C2: scores ~ N(0, 3), key lengths U{16..L}, grad_out ~ N(0, 1)."""
    g = rng(config)
    b, _, _, k = shape
    return {
        "scores": normal16(g, shape, 3.0),
        "key_lengths": g.integers(16, k + 1, size=b).astype(np.int32),
        "grad_out": normal16(g, shape, 1.0),
    }


def embedding_inputs(shape=C4, config=4, zipf_s=1.1):
    """C4 embedding inputs: Zipf(1.1) ids, token table, sinusoidal positions.

    The token table is drawn N(0, H^-1/2) so that s * E with s = sqrt(H) has
    unit scale (the usual Transformer initialisation); dy ~ N(0, 1).
    """
    g = rng(config, stream=1)
    h = shape.hidden
    return {
        "ids": zipf_ids(g, (shape.batch, shape.seq), shape.vocab, zipf_s),
        "tok_emb": normal16(g, (shape.vocab, h), h ** -0.5),
        "pos_emb": sinusoid_table(shape.seq, h),
        "grad_out": normal16(g, (shape.tokens, h), 1.0),
        "scale": float(np.sqrt(h)),
    }


CRITERION_ROW_CHUNK = 256
CRITERION_SMOOTHING = 0.1     # label smoothing of the Transformer-big translation setting
CRITERION_LOSS_SCALE = 4096.0  # fp16 loss scale: mean-over-tokens gradients stay representable


def criterion_targets(shape=C4, config=4, zipf_s=1.1):
    """Next-token targets for the C4 criterion: the same Zipf(1.1) law as the ids."""
    return zipf_ids(rng(config, stream=2), (shape.tokens,), shape.vocab, zipf_s)


def criterion_logits(r0, r1, shape=C4, config=4):
    """Rows [r0, r1) of the C4 logits [tokens, vocab], N(0, 1) in fp16.

    Rows come in chunks of CRITERION_ROW_CHUNK drawn from independent streams,
    so any row range can be regenerated on its own.
    """
    out = np.empty((r1 - r0, shape.vocab), np.float16)
    c0, c1 = r0 // CRITERION_ROW_CHUNK, (r1 - 1) // CRITERION_ROW_CHUNK
    for c in range(c0, c1 + 1):
        block = normal16(rng(config, stream=1000 + c), (CRITERION_ROW_CHUNK, shape.vocab), 1.0)
        lo, hi = max(r0, c * CRITERION_ROW_CHUNK), min(r1, (c + 1) * CRITERION_ROW_CHUNK)
        out[lo - r0:hi - r0] = block[lo - c * CRITERION_ROW_CHUNK:hi - c * CRITERION_ROW_CHUNK]
    return out


def adam_chunk(chunk, n=C5_CHUNK, config=5):
    """One chunk of the C5 workspace: p ~ N(0, 0.02), g ~ N(0, 1e-3).

    Chunks are drawn from independent streams so any one can be regenerated
    on its own.
    """
    g = rng(config, stream=100 + int(chunk))
    return normal16(g, (n,), 0.02), normal16(g, (n,), 1e-3)


ADAM_HYPER = dict(lr=1e-4, beta1=0.9, beta2=0.98, eps=1e-8, weight_decay=0.01,
                  grad_scale=1.0, decoupled_wd=True)
ADAM_STEPS = 10
