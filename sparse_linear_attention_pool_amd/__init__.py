"""SLA2 sparse-linear attention forward for MI355X (gfx950).

The compute path is the HIP library ``libsla2.so`` built from ``csrc/``; the
Python functions here only marshal arguments to its C entry points.
"""
