"""CPU oracle for the DSpark draft-sample-verify path.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
GPU kernels are checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or run it; the product
path (the HIP library and its Python binding) never does, and it shares no
code, table or constant generator with that path.

Precision: fp64 wherever the method is a plain definition (logits, bias,
softmax, Gumbel keys); float32 where a step is specified to be bit-exact on
both sides (the uniform map, the portable log2 of the exponential race, the
residual subtraction, the running survival product).

Modules
  philox   Philox4x32-10 counter-based generator and the uniform map.
  variates Gumbel noise, portable log2, exponential race (exact argmax).
  stages   The four stages: draft_logits, markov_sample, verify, admit,
           plus build_inverse_map and accept_prob (1 - total variation).

Pins (each checked by a ``-m "not gpu"`` test against something other than
the oracle itself) are listed in each function's docstring.  Functions with
no such pin are marked "parity unpinned" there.
"""
from . import philox, variates, stages  # noqa: F401
from .stages import (  # noqa: F401
    draft_logits, markov_sample, verify, admit, build_inverse_map,
    accept_prob, probs_from_logits, draft_probs,
)
