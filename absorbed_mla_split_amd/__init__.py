"""Folded split-KV absorbed-MLA decode for AMD MI355X (gfx950).

- ``binding``   ctypes binding of libamla.so (include/amla.h): plan, decode, combine.
- ``workloads`` seeded synthetic inputs (lengths, block tables, FP8 query and cache).
- ``build``     hipcc build of libamla.so.
"""
