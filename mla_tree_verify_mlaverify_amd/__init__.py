"""DDTree speculative-decode verify attention (absorbed MLA) for MI355X / gfx950.

The computation lives in libmlaverify.so (hand-written HIP kernels behind the C ABI
of include/mlaverify.h); this package only builds it and binds it to torch tensors.
"""

from .binding import (  # noqa: F401
    DEVERR_BAD_INDEX,
    DEVERR_BAD_PARENT,
    DEVERR_BAD_PREFIX,
    DEVERR_RELOCATE_CONFLICT,
    DEVERR_BAD_TREE_LEN,
    FLAG_NO_FASTPATH,
    LATENT_DIM,
    LIB_PATH,
    V_DIM,
    MlaVerifyError,
    Verifier,
    load_library,
    make_config,
    probe_gather,
    run_static,
    status_string,
    tree_masks,
    validate_config,
    workspace_bytes,
)
