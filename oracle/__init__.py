"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle (see oracle/oracle.py)."""
