"""libspecverify: batched speculative-decoding verification on MI355X (gfx950).

The HIP library (``libspecverify.so``, C ABI in ``include/specverify.h``) does
all of the work; ``binding`` marshals torch tensors into it: ``verify`` (one
verification step), ``sample`` (draws from processed distributions, e.g. the
draft model's), ``acceptance_rates`` (per-position sum_x min(p, q)),
``round_stats`` and ``DraftLengthMonitor`` (round statistics and the adaptive
draft length, on the device).
"""

from .binding import (  # noqa: F401
    TOTAL_FIELDS,
    DraftLengthMonitor,
    acceptance_rates,
    round_stats,
    sample,
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
