"""Plain fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP kernels or their host library.

Pages cited in this package (the reader has these pages):

* "Attention flash et question de longueur de séquence" (marketmaker.cc blog,
  French) -- sections "L'algorithme Flash Attention", "La récurrence softmax
  en ligne", "Passe arrière", "FA2 : parallélisme", "Le masquage causal".
* "Flash Attention" (ultralytics.com glossary, French) -- section
  "Fonctionnement de Flash Attention" and its PyTorch loop.
* "Почему Flash Attention быстрее" (sloger.press, Russian) -- sections
  "Проблема — трафик", "Online softmax".
* "FlashAttention: Fast and Memory-Efficient Exact Attention with
  IO-Awareness", reading guide (xyznot.com, Portuguese) -- sections
  "Problema e motivação", "Método" (incremental softmax equations and the
  four per-block steps, "Rastreamento Incremental do Softmax"),
  "Extensão: Block-Sparse FlashAttention".
* "Почему Flash Attention быстрее" (sloger.press) -- section "Что это
  изменило на практике" (decoding: a few queries against a long history).
* marketmaker.cc page, section "FA3 : Mécanique de la trémie", point 3 (FP8
  with incoherent processing: random rotation, then per-block quantisation).
* Dropout fused into the kernel: the reading guide's "Ideias centrais"
  ("Fusão de Kernels") and the marketmaker.cc page's `dropout_p` argument
  ("L'intégration est de huit lignes"); the mask comes from Philox-4x32-10
  (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
  SC 2011).

Every function in this package has at least one pin in
``tests/test_oracle_*.py`` that checks it against something other than
itself (closed forms, invariants, finite differences, an independent
library route, brute force, or the worked example one page prints).
No function is "parity unpinned".
"""

from .attention import (  # noqa: F401
    MASK_BLOCK,
    allowed,
    forward,
    forward_head,
    backward,
    backward_head,
    backward_head_sampled,
    backward_head_terms,
    rowsum_do_o,
)
from .decode import (  # noqa: F401
    combine,
    decode,
    decode_allowed,
    decode_head,
    split_partials,
)
from .dropout import (  # noqa: F401
    backward_head_dropout,
    backward_head_dropout_terms,
    dq_rows_dropout,
    forward_head_dropout,
    keep_mask,
    keep_scale,
    keep_threshold,
    philox,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    block_quantize,
    e4m3,
    fp8_forward,
    fp8_forward_head,
    hadamard,
    pow2_scale,
    rotate,
)
from .online import (  # noqa: F401
    merge_stats,
    online_softmax_normalised_each_step,
    online_softmax_deferred,
)
