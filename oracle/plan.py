"""Chunk plan of the overlap schedule (test infrastructure only).

Pure integer code, written from [TE#1344]'s option list:

* "method": ring_exchange (all-gather and reduce-scatter), pipeline (reduce-scatter only
  on the pages), bulk;
* "num_splits": number of chunks the GEMM is cut into; ignored for ring_exchange, where
  it is forced to the tensor-parallel size;
* "num_max_streams": compute streams = min(num_splits, num_max_streams), default 3;
* "aggregate": merge GEMM chunks two at a time when overlapping the all-gather;
* "atomic_gemm": one kernel loops over the chunks on the device instead of a host loop
  of per-chunk launches (same arithmetic, same chunks).

and from [TE#3564] "Implementation approach in the prototype": chunk views and byte
offsets are rebuilt from the ACTIVE first dimension T, never from the capacity.

Readings (the pages leave these open):

* chunk c of n covers rows [floor(c*T/n), floor((c+1)*T/n));
* aggregate pairs chunks {2u, 2u+1}; the last unit is a single chunk when n is odd;
  it applies to the all-gather side only;
* all-gather ring order: step i processes unit (home - i) mod U, home = rank // agg
  (each rank starts on its own chunk, then the ones received from its left neighbour);
* reduce-scatter ring order: step i processes chunk (rank + 1 + i) mod n, so a rank's
  own shard is the last one finished, as in a ring where each partial moves forward
  and its owner adds last;
* pipeline and bulk process units in natural order;
* the plan position j runs on compute stream j mod S; S is additionally capped by the
  library's stream-pool size when one is given.
"""

from dataclasses import dataclass

RING = "ring_exchange"
PIPELINE = "pipeline"
BULK = "bulk"
METHODS = (RING, PIPELINE, BULK)

DEFAULT_NUM_MAX_STREAMS = 3


# Order of the reduce-scatter sum (reduce-scatter side only):
#  "ascending" -- all tp partials summed at once, rounded to bf16 once;
#  "ring"      -- the sum a ring reduce-scatter computes, rounded to bf16 at every hop.
REDUCE_ORDERS = ("ascending", "ring")


@dataclass(frozen=True)
class OverlapCfg:
    method: str = RING
    num_splits: int = 1
    num_max_streams: int = DEFAULT_NUM_MAX_STREAMS
    aggregate: bool = False
    atomic_gemm: bool = False
    rank: int = 0
    reduce_order: str = "ascending"


@dataclass(frozen=True)
class Unit:
    pos: int      # position in execution order
    index: int    # unit index (after aggregation)
    row0: int     # first active row
    row1: int     # one past the last active row
    stream: int   # compute stream this position runs on


def effective_splits(cfg, tp):
    return tp if cfg.method == RING else cfg.num_splits


def chunk_rows(T, n):
    """Row ranges of the n chunks of an active T."""
    return [((c * T) // n, ((c + 1) * T) // n) for c in range(n)]


def num_streams(cfg, tp, stream_limit=None):
    s = min(effective_splits(cfg, tp), cfg.num_max_streams)
    if stream_limit is not None:
        s = min(s, stream_limit)
    return s


def build(T, tp, cfg, op, stream_limit=None):
    """Execution plan for one chunked GEMM call.

    op is "ag" (column-parallel, all-gather side) or "rs" (row-parallel, reduce-scatter
    side).  Returns the units in execution order.
    """
    if op not in ("ag", "rs"):
        raise ValueError(op)
    n = effective_splits(cfg, tp)
    if n < 1:
        raise ValueError("num_splits must be >= 1")
    chunks = chunk_rows(T, n)

    agg = 2 if (cfg.aggregate and op == "ag") else 1
    units = []
    for u in range((n + agg - 1) // agg):
        first, last = u * agg, min(u * agg + agg, n) - 1
        units.append((chunks[first][0], chunks[last][1]))
    U = len(units)

    if cfg.method == RING and op == "ag":
        home = cfg.rank // agg
        order = [(home - i) % U for i in range(U)]
    elif cfg.method == RING and op == "rs":
        order = [(cfg.rank + 1 + i) % U for i in range(U)]
    else:
        order = list(range(U))

    S = num_streams(cfg, tp, stream_limit)
    return [Unit(pos=j, index=u, row0=units[u][0], row1=units[u][1], stream=j % S)
            for j, u in enumerate(order)]
