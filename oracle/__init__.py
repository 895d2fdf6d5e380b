"""fp64 CPU oracle for the gated linear recurrences — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct reference that the HIP path
is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``gated_linear_recurrences_amd``) never imports, calls or links it, and it
shares no code with the HIP path: the two meet only in the seeded input
generators, which hold none of the method's arithmetic.

Sources (web pages; cited by title and section):
  * "Scrivere meglio nella memoria: gate e delta rule" (book.paithon.it,
    chapter on linear attention) - the recurrences, the gates, the delta rule,
    Gated DeltaNet, the online-regression reading and the transition table.
  * "Le architetture lineari: RetNet, RWKV, xLSTM" (book.paithon.it) - the
    three equivalent forms of retention (parallel, recurrent, chunkwise),
    Fig. 16.5 and its worked example.
  * "Riepilogo Tecnico: Attenzione Lineare Variazionale (VLA)" (gist.science) -
    variational linear attention: the Sherman-Morrison update of the inverse
    penalty, the normalised gating vector, the residual write and the ELU+1
    ratio readout.

Every function here is pinned by a ``-m "not gpu"`` test against something other
than itself (values the pages print, closed forms, invariants, brute force);
none is "parity unpinned".
"""

from .glr_oracle import (  # noqa: F401
    retention_recurrent,
    retention_quadratic,
    retention_chunkwise,
    scalar_recurrent,
    scalar_quadratic,
    scalar_chunkwise,
    gla_recurrent,
    gla_quadratic,
    gla_chunkwise,
    gdelta_recurrent,
    gdelta_quadratic,
    gdelta_chunkwise,
    decode_step,
    gdelta_decode_step,
    silu_l2,
    rms_norm,
    layer_norm,
    scalar_backward,
    gdelta_backward,
    retention_backward,
    gla_backward,
    vla_recurrent,
    vla_decode_step,
    elu1,
    forward_substitution,
)
