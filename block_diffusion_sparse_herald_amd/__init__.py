"""HERALD-style once-per-block sparse KV selection and block attention on MI355X (gfx950).

The compute path is the HIP library ``libherald.so`` (C ABI, include/herald.h);
``herald`` is its thin Python binding. ``inputs`` draws seeded synthetic workloads.
"""
