"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle of the selective scan (see oracle.py)."""
