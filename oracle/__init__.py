"""CPU oracle for the RecSA hot path -- test infrastructure only.

Imported by the tests, by ``__graft_entry__.smoke()`` and by the CPU
baseline leg of ``bench.py``; never by the GPU library or its binding.
"""
from . import recsa  # noqa: F401
