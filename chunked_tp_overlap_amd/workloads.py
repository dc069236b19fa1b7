"""Seeded synthetic workloads shared by the tests, the bench and the oracle's callers.

This module draws inputs and nothing else: it holds none of the method's arithmetic (no
GEMM, no reduction, no chunk plan, no offsets).  Values are drawn in float32 with numpy's
PCG64 generator and cast to bf16 with torch's CPU conversion; the resulting uint16 bit
patterns are what both the HIP path and the oracle receive.

Workload shapes follow the pages' layer shapes ([MLM#1240], "Why doesn't the hidden
dimension appear in initialize_ub()?": QKV ``[S,H] -> [S,3H/TP]``, MLP fc1
``[S,H] -> [S,2H/TP]``, fc2 back to ``[S,H]``) and THD packed-token microbatches whose
token count T varies ([TE#3564], "Problem").  The pages name no dataset; these seeded
draws are the workloads.
"""

from dataclasses import dataclass, field

import numpy as np

CANARY = 0x7FA5  # NaN pattern used to fill bytes that must stay untouched


def to_bf16_bits(x):
    """float array -> uint16 bf16 patterns via torch's CPU cast (round to nearest even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bits(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return to_bf16_bits(x)


def uniform_bits(rng, shape, lo=-1.0, hi=1.0):
    return to_bf16_bits(rng.uniform(lo, hi, size=shape).astype(np.float32))


def integer_bits(rng, shape, lo=-2, hi=2):
    """Integer values in [lo, hi] (exact in bf16)."""
    return to_bf16_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32))


def const_bits(shape, value):
    return to_bf16_bits(np.full(shape, value, dtype=np.float32))


# -- workload configurations ---------------------------------------------------------

@dataclass
class Workload:
    """One workload: registration shape, GEMM shape, overlap options, T set, seeds."""
    name: str
    capacity: int
    hidden: int
    tp: int
    op: str                  # "ag" or "rs"
    n_cols: int              # AG: output columns N; RS: output columns = hidden
    k: int                   # reduction size: AG: hidden; RS: full K (split into tp slices)
    method: str
    num_splits: int
    num_max_streams: int = 3
    aggregate: bool = False
    a_dist: str = "normal"   # activations: "normal" N(0,1) or "uniform" U[-1,1]
    w_std: float = 0.02      # weights N(0, w_std) (std, not variance) when a_dist == normal
    seed: int = 1000
    description: str = ""
    extra: dict = field(default_factory=dict)

    def seeds(self):
        """Independent generators for (activations, weights, token counts)."""
        ss = np.random.SeedSequence(self.seed)
        return [np.random.default_rng(s) for s in ss.spawn(3)]

    def flops(self, T):
        return 2.0 * T * self.k * self.n_cols


def tiny_ag():
    return Workload(
        name="tiny_ag", capacity=512, hidden=256, tp=2, op="ag", n_cols=384, k=256,
        method="ring_exchange", num_splits=2, num_max_streams=3, a_dist="uniform",
        seed=1001,
        description="tiny column-parallel AG-GEMM: capacity 512, hidden 256, tp 2, T 256, "
                    "W [256,384], ring, bf16 U[-1,1]")


def tiny_rs():
    return Workload(
        name="tiny_rs", capacity=512, hidden=256, tp=2, op="rs", n_cols=256, k=256,
        method="ring_exchange", num_splits=2, num_max_streams=3, a_dist="uniform",
        seed=1001,
        description="tiny row-parallel RS: K=256 in 2 slices of 128, out [256,256], "
                    "2 shards [128,256], bf16 U[-1,1]")


def qkv():
    return Workload(
        name="qkv_ag", capacity=8192, hidden=4096, tp=8, op="ag", n_cols=1536, k=4096,
        method="ring_exchange", num_splits=8, num_max_streams=3, seed=1002,
        description="QKV column-parallel AG-GEMM: capacity 8192, hidden 4096, tp 8, "
                    "W [4096,1536], 8 ring chunks, 3 streams, 32 THD packs")


def fc1():
    return Workload(
        name="fc1_ag", capacity=16384, hidden=4096, tp=8, op="ag", n_cols=3584, k=4096,
        method="ring_exchange", num_splits=8, num_max_streams=3, aggregate=True, seed=1003,
        description="SwiGLU fc1 column-parallel AG-GEMM: capacity 16384, hidden 4096, tp 8, "
                    "W [4096,3584], 8 chunks aggregated 2x, 3 streams, 16 microbatches")


def fc2():
    return Workload(
        name="fc2_rs", capacity=16384, hidden=4096, tp=8, op="rs", n_cols=4096, k=14336,
        method="pipeline", num_splits=4, num_max_streams=3, seed=1004,
        description="MLP fc2 row-parallel RS-GEMM: capacity 16384, hidden 4096, K 14336 in "
                    "8 slices of 1792, pipeline, 4 chunks, 8 shards [T/8,4096]")


def gqa_bulk():
    return Workload(
        name="gqa_bulk_ag", capacity=32768, hidden=8192, tp=8, op="ag", n_cols=1280, k=8192,
        method="bulk", num_splits=8, num_max_streams=3, seed=1005,
        description="GQA QKV AG-GEMM bulk: capacity 32768, hidden 8192, tp 8, W [8192,1280], "
                    "8 chunks, T = 1024 + 1016 k on one buffer")


ALL = {w().name: w for w in (tiny_ag, tiny_rs, qkv, fc1, fc2, gqa_bulk)}


# -- token-count (T) draws ---------------------------------------------------------------

def qkv_pack_tokens(rng, n_micro=32, capacity=8192, lo=128, hi=4096, multiple=8):
    """THD packs: sequence lengths uniform on [lo, hi] are appended until the next one
    would exceed the capacity (that one is dropped); T is then rounded down to a
    multiple of 8.  Returns (T values, per-pack sequence lengths)."""
    Ts, packs = [], []
    for _ in range(n_micro):
        lens, t = [], 0
        while True:
            ln = int(rng.integers(lo, hi + 1))
            if t + ln > capacity:
                break
            lens.append(ln)
            t += ln
        Ts.append((t // multiple) * multiple)
        packs.append(lens)
    return Ts, packs


def fc1_tokens(rng, n_micro=16, lo=1024, hi=16384, multiple=8):
    """T uniform over the multiples of 8 in [lo, hi]."""
    return [int(multiple * rng.integers(lo // multiple, hi // multiple + 1))
            for _ in range(n_micro)]


FC2_TOKENS = (2048, 6144, 12280, 16384)


def gqa_tokens(include_capacity=True):
    """T = 1024 + 1016 k for k = 0..31 (1024 ... 32520); 32768 appended as an extra
    point (it is not on the 1016-step grid)."""
    ts = [1024 + 1016 * k for k in range(32)]
    if include_capacity:
        ts.append(32768)
    return ts


def tokens_for(w, rng=None):
    if rng is None:
        rng = w.seeds()[2]
    if w.name in ("tiny_ag", "tiny_rs"):
        return [256]
    if w.name == "qkv_ag":
        return qkv_pack_tokens(rng)[0]
    if w.name == "fc1_ag":
        return fc1_tokens(rng)
    if w.name == "fc2_rs":
        return list(FC2_TOKENS)
    if w.name == "gqa_bulk_ag":
        return gqa_tokens()
    raise KeyError(w.name)


def activations(w, rows, rng=None):
    """``[rows, k]`` activation patterns for workload w (AG: the UserBuffer rows)."""
    if rng is None:
        rng = w.seeds()[0]
    if w.a_dist == "uniform":
        return uniform_bits(rng, (rows, w.k))
    return normal_bits(rng, (rows, w.k), 1.0)


def weights(w, rng=None):
    """``[k, n_cols]`` weight patterns for workload w."""
    if rng is None:
        rng = w.seeds()[1]
    if w.a_dist == "uniform":
        return uniform_bits(rng, (w.k, w.n_cols))
    return normal_bits(rng, (w.k, w.n_cols), w.w_std)
