"""CPU oracle for MLA absorbed decode -- test infrastructure.

Only tests/, the smoke check in __graft_entry__ and the benchmark's CPU
baseline may import anything under oracle/. The GPU product path never does.
"""
