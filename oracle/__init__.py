"""CPU oracle for the QSA hot path -- test infrastructure only.

Imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg.
The library never imports it.
"""
