"""The five synthetic decode workloads, as plain data.

Each workload is one decode step of multi-head latent attention on a batch of
sequences: the queries of T new tokens per sequence, a paged latent cache that
already holds N rows per sequence, and the per-head up-projections W^UK and
W^UV.  The step appends the T new rows and then attends over N + T rows.

Dimensions follow the pages:
  * DeepSeek-V3 latent width d_c = 512 and decoupled rotary key d^R_h = 64
    ("Attention, Part 2: MQA, GQA and MLA", section "The MLA equations").
  * The V2-scale head layout n_h = 128, d_h = 40 ("Multi-head latent attention
    (MLA)", section 2 "Down-projection to a latent").
  * Batches shaped after the 8 conversations x 4,096 tokens timing ("Attention,
    Part 2", section "Does a smaller cache make writing faster?"), variable
    length serving (the FlashMLA entry of "Research on MLA"), and 128K contexts
    ("Attention, Part 2", section "The impact, and where you meet it").

This module holds no attention arithmetic; it only describes shapes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int                 # sequences in the batch
    T: int                 # new query tokens per sequence
    H: int                 # query heads n_h
    d_c: int               # latent width
    d_r: int               # decoupled rotary key width d^R_h
    d_n: int               # per-head content query/key width (rows of W^UK)
    d_v: int               # per-head value width (rows of W^UV)
    N: int                 # rows cached per sequence before the step (max if var_len)
    dtype: str             # "f32" or "bf16": cache, queries and weights
    block_size: int = 64   # tokens per cache page
    causal: bool = True    # new tokens see the cache and the new tokens before them
    table: str = "sequential"   # "sequential" or "permuted" page placement
    var_len: bool = False  # per-sequence N drawn uniformly from [1, N]
    outlier_frac: float = 0.0   # fraction of cached rows scaled by outlier_scale
    outlier_scale: float = 1.0
    d_model: int = 0       # model width d, for the producer step (0: no source gives it)

    @property
    def W(self) -> int:
        """Width of one cached row: latent plus rotary key."""
        return self.d_c + self.d_r

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d_n + d_r), as the page-3 absorbed path divides."""
        return 1.0 / math.sqrt(self.d_n + self.d_r)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# 1: tiny fp32, identity page table (a contiguous cache in memory)
TINY = Workload(name="tiny_f32", seed=1, B=1, T=1, H=16, d_c=64, d_r=16, d_n=32,
                d_v=32, N=128, dtype="f32")
# 2: DeepSeek-V3 shape, 16 sequences x 4,096 cached rows
V3 = Workload(name="v3_decode", seed=2, B=16, T=1, H=128, d_c=512, d_r=64, d_n=128,
              d_v=128, N=4096, dtype="bf16")
# 3: variable-length serving batch, permuted pages
VARLEN = Workload(name="varlen_serving", seed=3, B=64, T=1, H=128, d_c=512, d_r=64,
                  d_n=128, d_v=128, N=32768, dtype="bf16", table="permuted",
                  var_len=True)
# 4: 128K context, 1% of cached rows x8
LONG = Workload(name="long_128k", seed=4, B=4, T=1, H=128, d_c=512, d_r=64, d_n=128,
                d_v=128, N=131072, dtype="bf16", outlier_frac=0.01, outlier_scale=8.0)
# 5: V2-scale heads, 4 new tokens per sequence with a causal mask among them
# (model width d = 5120 from the V2-scale configuration of "Multi-head latent
# attention (MLA)", section 1)
V2_MULTI = Workload(name="v2_multi_token", seed=5, B=32, T=4, H=128, d_c=512, d_r=64,
                    d_n=40, d_v=40, N=8192, dtype="bf16", d_model=5120)

ALL = (TINY, V3, VARLEN, LONG, V2_MULTI)

# Beyond the five decode configs: a chunk of prefill -- 512 new tokens per
# sequence attend causally to 3,584 cached rows and to each other, through the
# same absorbed path (the pages' absorbed code runs exactly this with T > 1).
# No page gives a prefill shape; V3 widths, 4 sequences, 4,096 rows after.
PREFILL = Workload(name="prefill_chunk", seed=6, B=4, T=512, H=128, d_c=512, d_r=64,
                   d_n=128, d_v=128, N=3584, dtype="bf16")
EXTRA = (PREFILL,)

BY_NAME = {w.name: w for w in ALL + EXTRA}
