"""MI355X-native ragged paged attention.

The compute path lives in the HIP/C-ABI library libragged_attn.so; this
package is a thin ctypes binding over it (torch supplies device memory and
the current HIP stream) plus the seeded input generators in ``inputs``.
"""
from .binding import (  # noqa: F401
    RaError,
    forward,
    lib_path,
    load_library,
    validate_metadata,
    workspace_bytes,
)
