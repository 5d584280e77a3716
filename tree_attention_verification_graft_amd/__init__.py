"""libgraft: the prune-then-graft speculative-decoding step on one MI355X.

`binding` exposes the C ABI's calls under the same names (ctypes, marshalling
only); `pipeline.DeviceStep` allocates buffers with torch and runs one step.
Importing this package loads the built HIP library and fails if it is absent.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    GraftError, graft_accept, graft_accept_workspace_size, graft_build_tree,
    graft_last_error, graft_tree_attention, graft_tree_attention_workspace_size,
    graft_update_adjacency, graft_update_adjacency_workspace_size, graft_version,
)
