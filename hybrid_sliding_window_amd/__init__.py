"""hybrid_sliding_window_amd: the attention core of a hybrid sliding-window
transformer (MiMo-V2.6 shapes) as hand-written gfx950 HIP behind a C ABI.

- ``hsw``: ctypes binding of libhsw.so (imports fail if it is not built)
- ``workloads``: seeded synthetic inputs (no arithmetic of the method)
- ``build``: compiles libhsw.so in place
"""
