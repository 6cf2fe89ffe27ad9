"""CPU fp64 oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check (__graft_entry__.smoke) and the
benchmark's CPU-baseline leg; never by the HIP library or its binding.

Pin status: every function here is pinned by a CPU test against something
other than itself (brute force, closed forms, invariants, a library routine,
or values the pages print); none is "parity unpinned".
"""
