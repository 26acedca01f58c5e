"""MI355X (gfx950) DSA decode step: indexer scores, exact top-k, sparse attention.

The work runs in hand-written HIP kernels inside ``libdsa.so`` (C ABI declared in
``include/dsa.h``). ``binding`` marshals torch tensors into those calls; it is
imported on first use so that ``inputs`` can be used without the library.
"""
import importlib

__all__ = ["dsa_index_scores", "dsa_topk_select", "dsa_sparse_attn", "dsa_decode_step",
           "dsa_workspace_size", "dsa_status_string", "dsa_read_stats", "DSAError",
           "FLAG_FORCE_FALLBACK", "library_path", "build", "new_workspace", "load_library"]


def __getattr__(name):
    if name in __all__:
        return getattr(importlib.import_module(".binding", __name__), name)
    raise AttributeError(name)
