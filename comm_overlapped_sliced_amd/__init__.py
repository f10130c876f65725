"""libflashovl: the Flash-Overlap hot path (Flash-AG / Flash-RS) on MI355X (gfx950).

The compute path is the C-ABI shared library ``libflashovl.so`` built from ``csrc/``; this
package holds its thin ctypes binding (``flashovl``), the workload table (``configs``) and the
seeded input generators (``inputs``). Importing the package loads nothing; the library is
opened on first use and a missing library is an error, never a fallback.
"""
