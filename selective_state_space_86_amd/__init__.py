"""MI355X (gfx950) selective state-space scan (S6): Python binding of libss.

Every step of the scan runs in the HIP kernels of ``libss.so``; this package only
marshals torch device tensors into the C ABI declared in ``include/ss.h``
(``ss_fwd``, ``ss_fwd_conv``, ``ss_step``, ``ss_bwd``, ``ss_proj``). The library is loaded on first use and a missing or
unloadable build raises: there is no fallback path.
"""
from ._binding import (SSError, bwd, bwd_workspace_size, fwd, fwd_conv, fwd_noalloc, fwd_plain,  # noqa: F401
                       fwd_workspace_size, lib_path, load_library, proj, proj_conv, step,
                       workspace_status)

__all__ = ["fwd", "fwd_plain", "fwd_noalloc", "fwd_conv", "fwd_workspace_size", "workspace_status", "step", "bwd",
           "bwd_workspace_size", "proj", "proj_conv", "SSError", "load_library", "lib_path"]
