"""CPU oracle for H2O budgeted attention: test infrastructure only.

Importable by the tests, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg; never by the product path.  See ``h2o_oracle`` for the
definitions and the readings it takes.
"""
from .h2o_oracle import (  # noqa: F401
    NO_PATTERN, TIE_RTOL, ParityMismatch, Pattern, PrefillScores, Rope, UnitCache, default_scale, global_scores,
    prefill_keep,
    prefill_output, prefill_scores, run_unit, run_unit_global, softmax,
)
