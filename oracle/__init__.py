"""Plain fp64 CPU oracle for EntmaxKV paged decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the test suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code, constants or helpers with the HIP library.

Parity status of each function is stated in ``entmax_oracle``'s header.
"""
from .entmax_oracle import *  # noqa: F401,F403
