"""Identity Hyper-Connections residual path for MI355X (gfx950).

The GPU work runs in ``libhc.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/hc.h``); this package holds the thin ctypes binding
(``hyper_connections_amd.hc``) and the seeded synthetic workloads
(``hyper_connections_amd.workloads``).  The binding loads the library on first
use and raises if it is missing: there is no CPU fallback.
"""
