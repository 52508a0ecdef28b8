"""Float64 CPU oracle of the RSM mixer.

TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code with the
HIP library (``sparse_routed_slot_amd``) and never imports it.
"""
