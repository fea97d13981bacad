"""Double-precision CPU oracle for the frame-wise GDN forward recurrence.

Test infrastructure only: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use it; the product path never does.
"""
