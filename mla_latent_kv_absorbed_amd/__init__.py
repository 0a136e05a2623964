"""MI355X-native absorbed MLA decode attention over a paged latent KV cache.

The compute runs in hand-written HIP kernels for gfx950 behind the C ABI of
include/mla.h (libmla.so, built in this directory); this package only
marshals arguments.  See `decode`, `make_plan`, `lse_combine`, `prepare`.
"""

from ._binding import (  # noqa: F401
    KV_BF16,
    KV_FP4,
    KV_FP8,
    KV_MXFP8,
    DecodeDesc,
    MlaError,
    check_table,
    Plan,
    decode,
    decode_noalloc,
    library_path,
    load_library,
    lse_combine,
    lse_combine_project,
    make_desc,
    make_plan,
    plan_max_bytes,
    prepare,
    status_string,
)
