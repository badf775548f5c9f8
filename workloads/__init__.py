"""Seeded synthetic inputs for the MXFP4 quantizer and GEMMs.

Shared by the GPU path's tests/bench and the oracle's tests; it holds none of
the method's arithmetic (no scaling, rounding, transform or GEMM), only the
random inputs: tensors, the Hadamard sign mask and the stochastic-rounding
seed (random numbers the method draws are passed in as inputs).

Every stream is ``np.random.default_rng(SeedSequence([cfg_id, stream_id, ...]))``
with cfg_id 1..6 for the workloads (tiny, quantize-only, dense fprop,
wgrad, MoE grouped, dgrad) and stream ids 0 = A/X, 1 = B/W/dY, 2 = outlier
positions, 3 = Hadamard sign mask, 4 = Philox seed, 5 = MoE routing.
bfloat16 tensors are made from float32 by round-to-nearest-even (torch's CPU
cast), so every consumer sees identical bits.

The shapes and distributions stand in for the pages' GPT-OSS-20B workloads
(hidden size 2880, expert width 5760, 32 experts, top-4 routing); no model
weights or datasets are used.
"""

import numpy as np
import torch

CFG_TINY, CFG_QUANT, CFG_FPROP, CFG_WGRAD, CFG_MOE, CFG_DGRAD = 1, 2, 3, 4, 5, 6
S_A, S_B, S_OUTLIER, S_MASK, S_SEED, S_ROUTE = 0, 1, 2, 3, 4, 5


def rng(cfg_id, stream_id, *extra):
    return np.random.default_rng(np.random.SeedSequence([cfg_id, stream_id, *extra]))


def to_bf16(x):
    """float32 numpy -> bfloat16 CPU tensor (RNE)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def normal_f32(cfg_id, stream_id, shape, std=1.0, *extra):
    g = rng(cfg_id, stream_id, *extra)
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def rht_mask(cfg_id):
    """32-bit random sign mask for the Hadamard transform."""
    return int(rng(cfg_id, S_MASK).integers(0, 2**32, dtype=np.uint64))


def philox_seed(cfg_id):
    """64-bit Philox key for stochastic rounding."""
    return int(rng(cfg_id, S_SEED).integers(0, 2**64 - 1, dtype=np.uint64, endpoint=True))


def student_t_outliers(rows, cols, cfg_id=CFG_QUANT, nu=3.0, frac=1e-3, factor=100.0):
    """Student-t(nu) values with a fraction `frac` of entries, chosen uniformly
    without replacement, multiplied by `factor`; returns a bf16 CPU tensor."""
    x = rng(cfg_id, S_A).standard_t(nu, size=(rows, cols)).astype(np.float32)
    n = rows * cols
    k = int(round(frac * n))
    if k:
        pos = rng(cfg_id, S_OUTLIER).choice(n, size=k, replace=False)
        x.reshape(-1)[pos] *= np.float32(factor)
    return to_bf16(x)


def tiny(m=256, k=512, n=256):
    """Tiny case: A [m, k] and B [k, n], float32 N(0, 1)."""
    return (normal_f32(CFG_TINY, S_A, (m, k)), normal_f32(CFG_TINY, S_B, (k, n)))


def fprop(tokens=16384, k=2880, n=5760):
    """Dense fprop: X [tokens, k] bf16 N(0,1); W [k, n] bf16 N(0, 0.02)."""
    x = to_bf16(normal_f32(CFG_FPROP, S_A, (tokens, k)))
    w = to_bf16(normal_f32(CFG_FPROP, S_B, (k, n), 0.02))
    return x, w


def wgrad(tokens=16384, k=2880):
    """Wgrad: dY [tokens, k] bf16 N(0, 1e-3); X [tokens, k] bf16 N(0, 1)."""
    dy = to_bf16(normal_f32(CFG_WGRAD, S_B, (tokens, k), 1e-3))
    x = to_bf16(normal_f32(CFG_WGRAD, S_A, (tokens, k)))
    return dy, x


def dgrad(tokens=16384, k=2880, n=5760):
    """Dgrad of the dense layer: dY [tokens, n] bf16 N(0, 1e-3) and the fprop
    weight W [k, n] (the same tensor as fprop()'s)."""
    dy = to_bf16(normal_f32(CFG_DGRAD, S_B, (tokens, n), 1e-3))
    w = to_bf16(normal_f32(CFG_FPROP, S_B, (k, n), 0.02))
    return dy, w


def moe_routing(tokens=16384, experts=32, topk=4, s=1.1, seed=0):
    """Zipf(s) expert popularity over a seeded permutation of the experts; each
    token draws `topk` distinct experts by Gumbel-top-k on log p.

    Returns (token_of_row int64 [tokens*topk], offsets int32 [experts+1]):
    rows grouped by expert (ascending), tokens ascending within an expert."""
    g = rng(CFG_MOE, S_ROUTE, seed)
    ranks = np.arange(1, experts + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    perm = g.permutation(experts)             # expert id of popularity rank r
    logp = np.empty(experts)
    logp[perm] = np.log(p)
    gumbel = g.gumbel(size=(tokens, experts))
    choice = np.argsort(-(logp[None, :] + gumbel), axis=1, kind="stable")[:, :topk]
    tok = np.repeat(np.arange(tokens), topk)
    exp = choice.reshape(-1)
    order = np.lexsort((tok, exp))
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return tok[order], offsets


def moe_tokens(tokens=16384, k=2880):
    """Token activations X [tokens, k] float32 N(0, 1) (gathered per expert by the caller)."""
    return normal_f32(CFG_MOE, S_A, (tokens, k))


def moe_expert_weight(e, k=2880, n=5760):
    """Expert e's weight W_e [k, n] as float32 N(0, 0.02), its own stream."""
    return normal_f32(CFG_MOE, S_B, (k, n), 0.02, e)
