"""libmoda: the Mixture-of-Depths Attention operator on MI355X (gfx950).

The operator runs in hand-written HIP kernels behind the C ABI declared in
include/moda.h (libmoda.so, built in-tree).  ``binding`` is the ctypes layer
with the same entry-point names; ``inputs`` holds the seeded synthetic
workloads.  Importing the package does not load the library; the first call
does, and raises if libmoda.so has not been built.
"""
from .binding import (DepthKVCache, ModaError, Problem, bwd, decode, depth_append, fwd, load,
                      moda_attention, moda_bwd, moda_bwd_workspace_bytes, moda_fwd,
                      moda_fwd_chunk_tokens, moda_pack_depth, pack_depth, problem, problem_for)

__all__ = ["DepthKVCache", "ModaError", "Problem", "bwd", "decode", "depth_append", "fwd", "load",
           "moda_attention", "moda_bwd", "moda_bwd_workspace_bytes", "moda_fwd",
           "moda_fwd_chunk_tokens", "moda_pack_depth", "pack_depth", "problem", "problem_for"]
