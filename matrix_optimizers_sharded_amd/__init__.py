"""MI355X-native owner-local Muon step and Sign-Muon tail.

The compute lives in libmatopt.so (hand-written HIP for gfx950 behind a C ABI,
declared in include/matopt.h).  This package is a thin ctypes binding over it:
argument marshalling only, with PyTorch used for device memory and streams.
Importing the package does not load the library; the first call does, and raises
MatoptError if the library is missing.
"""

from .binding import (  # noqa: F401
    MatoptError,
    load_library,
    library_path,
    muon_step_batched,
    muon_step_batched_noalloc,
    muon_step_apply,
    ns_orthogonalize,
    sign_pack,
    sign_pack_batched,
    sign_vote,
    sign_unpack,
    sign_apply,
    plan_owners,
    workspace_bytes,
    version,
    profile_begin,
    profile_end,
    Workspace,
    MO_F32,
    MO_BF16,
    NOALLOC_SCRATCH_BYTES,
)
