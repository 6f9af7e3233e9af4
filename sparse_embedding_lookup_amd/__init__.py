"""MI355X-native sparse front end of a CTR ranking model.

The compute path is the C-ABI library ``libctr.so`` (hand-written HIP for gfx950) reached
through :mod:`sparse_embedding_lookup_amd.ctr`.  Importing the package loads nothing;
``workloads`` holds the seeded synthetic inputs.
"""
__all__ = ["ctr", "workloads"]
