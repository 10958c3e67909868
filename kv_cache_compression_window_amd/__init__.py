"""MI355X (gfx950) KV-cache scoring and pruning.

The compute path is the C-ABI library ``libkvc.so`` built from ``csrc/``;
``binding`` marshals torch tensors into its calls.  ``synth`` holds the
seeded synthetic inputs and ``configs`` the workloads.  Importing this
package does not load the library; ``from kv_cache_compression_window_amd
import binding`` does, and fails loudly if it is not built.
"""
__all__ = ["configs", "synth"]
