"""Build-if-missing helper for the tests (the library is built in-tree)."""

import os


def ensure_built():
    from structured_sparse_state_pdssm_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    return b.LIB
