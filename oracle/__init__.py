"""CPU oracle for the FlashAttention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
helpers with the HIP library under ``exact_attention_101_amd/``.

Everything here is plain, slow and written to be read against the pages:

* ``attention``  -- exact scaled-dot-product attention in float64 with the
  full N x N score matrix and a two-pass softmax (max pass, then exp/sum
  pass).  This is the "classic" computation that the FlashAttention v1 post
  (DeepSchool #630), sections «Проблема базового attention» and
  «Онлайн-Softmax», says the tiled method reproduces exactly.
  ``attention_kv`` is the same with Nq queries against Nk keys (decode,
  bottom-right causal alignment); ``attention_varlen`` runs it per sequence
  of a variable-length batch, with an optional sliding window;
  ``attention_masked`` takes an arbitrary boolean visibility mask.
* ``attention_bwd`` -- the exact gradients dQ, dK, dV of the same
  definition for a given dO, with the softmax recomputed (the pages name
  recomputation, FlashAttention-3 summary, «Resumo do FlashAttention», and
  the backward pass's shared-memory bottleneck, FlashAttention-4 page,
  paragraph 2, but give no formulas).
* ``fp8``        -- OCP e4m3 ("e4m3fn") encode/decode from the format's
  definition and per-tensor quantisation, for the low-precision path of the
  FlashAttention-3 summary (GeekNews), section «Novos recursos de hardware
  da GPU Hopper» (FP8) and «Baixa precisão ...».
* ``hadamard``   -- Sylvester-Hadamard matrix and the random-sign orthonormal
  rotation used for "incoherent processing" in the FlashAttention-3 summary,
  section «Baixa precisão: redução do erro de quantização com processamento
  incoerente».

Parity status of each function is stated in its module header.
"""

from .attention import (  # noqa: F401
    attention,
    attention_kv,
    attention_masked,
    attention_rows,
    attention_varlen,
)
from .attention_bwd import (  # noqa: F401
    attention_backward,
    attention_backward_sampled,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    e4m3_table,
    quantize_per_tensor,
)
from .hadamard import rotate, sylvester  # noqa: F401
