"""Closed-form tree verification for Gated DeltaNet layers on AMD MI355X (gfx950).

The compute path is libbole.so (hand-written HIP kernels behind the C ABI in
include/bole.h); this package is its thin Python binding plus device-buffer
plumbing.  Importing it does not load the library; the first call does, and
fails loudly if the library has not been built.
"""

from .bole import (  # noqa: F401
    BOLE_BF16, BOLE_F32, ERR_BAD_ACCEPT, ERR_BAD_PARENT, ERR_BAD_SLOT, ERR_CYCLE,
    ERR_TREE_SIZE, MAX_TREE, BoleError, bole_commit_path, bole_factor_gc, bole_factor_verify,
    bole_conv_commit, bole_gc_workspace_bytes, bole_status_string, bole_tree_conv, bole_tree_prep,
    bole_tree_verify, bole_commit_tree_verify, bole_verify, bole_verify_neumann, bole_factor_inverse, bole_verify_inverse,
    bole_forest_build, bole_forest_build_noalloc, bole_forest_workspace_bytes, lib,
)
from .runner import BucketedRound, ForestBuilder, Topology, TreeRound  # noqa: F401

__all__ = [
    "bole_tree_prep", "bole_factor_gc", "bole_verify", "bole_factor_verify", "bole_tree_verify",
    "bole_commit_tree_verify", "bole_verify_neumann", "bole_factor_inverse", "bole_verify_inverse",
    "bole_commit_path", "bole_tree_conv", "bole_conv_commit", "bole_forest_build",
    "bole_forest_build_noalloc",
    "bole_forest_workspace_bytes", "ForestBuilder", "BucketedRound",
    "bole_gc_workspace_bytes", "bole_status_string", "BoleError", "TreeRound", "Topology", "lib",
]
