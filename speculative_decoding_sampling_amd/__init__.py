"""libspecverify: batched speculative-decoding verification on MI355X (gfx950).

The HIP library (``libspecverify.so``, C ABI in ``include/specverify.h``) does
all of the work; ``binding.verify`` marshals torch tensors into it.
"""

from .binding import (  # noqa: F401
    PATH_BONUS,
    PATH_EOS,
    PATH_ERROR,
    PATH_REJECT,
    SpecVerifyError,
    library_path,
    load_library,
    status_string,
    verify,
    workspace_bytes,
)
