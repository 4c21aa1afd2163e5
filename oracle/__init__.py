"""CPU oracle for the low-bit dequant-GEMM path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything under ``oracle/``.

See ``oracle/ddg_oracle.py``, ``oracle/pd_oracle.py``, ``oracle/rpbh_oracle.py`` and
``oracle/fp4_oracle.py`` for the definitions and their citations.
"""
from .ddg_oracle import *  # noqa: F401,F403
from .pd_oracle import *  # noqa: F401,F403
from .rpbh_oracle import *  # noqa: F401,F403
from . import fp4_oracle as fp4  # noqa: F401  (names overlap the integer path)
