"""shared_history_candidate_amd: one-history-to-many-candidates cross-attention
for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libxattn.so`` (hand-written HIP);
``shared_history_candidate_amd.xattn`` is its thin ctypes binding and
``shared_history_candidate_amd.workloads`` the seeded input generators.
Importing the package loads nothing native; the binding loads the library on
first use and raises if it has not been built.
"""
__all__ = ["xattn", "workloads", "build"]
