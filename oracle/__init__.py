"""Plain CPU oracle for the MSA routing + sparse-attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``latent_memory_long_amd``) never imports it and shares no code,
tables or helpers with it.

Everything here is NumPy float64 and follows the written definition of each
step; see ``oracle.msa_oracle`` for the functions and their citations.
"""
from .msa_oracle import *  # noqa: F401,F403
