"""Plain, slow, fp64 CPU oracle for the Ulysses sequence-parallel hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (the HIP library and its Python binding) never
does, and the two share no code: no kernels, helpers, tables or constants.

Contents
--------
``exchange``   the emulated all-to-all exchanges as explicit per-rank
               send/receive loops (sequence shard -> head shard and back).
``attention``  exact softmax attention, forward (O and logsumexp) and
               backward (dQ, dK, dV), with causal and key-validity masks and
               grouped-query heads, as a two-pass softmax over materialised
               fp64 score rows.
``rope``       rotary position embedding at global positions before the first
               exchange.
``loss``       the loss aggregated over shards, weighted by valid tokens.
``proj``       the QKV projection before the first exchange and the output
               projection after the second.
``ring``       the ring-attention alternative: block attention and the exact
               logsumexp merge over the P hops.

Sources (web pages; cited by title and section):
  [ALST]  "Paralelismul de Secvență Ulysses: Antrenarea modelelor AI cu
          contexte de un milion de token-uri" (world.tibi.club)
  [HFSUM] "Ulysses 序列平行化：突破百萬標記長上下文的訓練瓶頸"
          (agents-report.net)
  [SWIFT] "ms-swift性能优化：Ulysses并行技术降低长文本显存" (hotelren.com)
"""
from . import exchange, attention, rope, loss, ring, proj  # noqa: F401
from .exchange import shard, unshard, seq2head, head2seq, check_constraints  # noqa: F401
from .attention import (  # noqa: F401
    attn_fwd, attn_bwd, attn_bwd_sampled, pipeline_fwd, pipeline_bwd, kv_head_of,
)
