"""CPU oracle of one DMTP speculative-decoding round -- TEST INFRASTRUCTURE.

This package is a plain, slow, float64 NumPy statement of what the round
computes, written from the pages (the DMTP blog "DMTP: A Better First Token
for Block Drafting via MTP", the "DFlash vs MTP" article and the colibri
speculative-decoding notes).  It exists to check the HIP library and for
nothing else: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``mtp_block_draft_amd``) never imports, links or calls anything here, and
this package never imports the product path; the two share only the seeded
input draws of ``dmtp_synth``.

Modules
  numerics  bf16 rounding, RMSNorm, RoPE, softmax, attention (definitions)
  philox    the Philox4x64-10 counter-based generator and Gumbel noise
  dmtp      the four steps of a round and the round itself
"""
from . import numerics, philox, dmtp  # noqa: F401
from .dmtp import run_round, RoundResult  # noqa: F401
