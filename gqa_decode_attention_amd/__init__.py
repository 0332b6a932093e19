"""MI355X (gfx950) grouped-query attention decode step.

Python face of the HIP library ``libgqa_decode.so`` (C ABI in
``include/gqa_decode.h``): ``append`` writes each sequence's new key/value at
slot ``lengths[b]`` of a fixed-capacity cache, ``attend`` runs length-masked
GQA attention over the cache, and ``step`` does both in one call.  torch is
used for device memory and streams only.
"""
from ._lib import (  # noqa: F401
    BF16,
    EXPORTS,
    F32,
    LIB_PATH,
    Desc,
    GqaError,
    MapT,
    append,
    append_mapped,
    attend,
    attend_mapped,
    check_lengths,
    desc_for,
    get_plan,
    lib,
    make_desc,
    step,
    step_mapped,
    workspace_size,
)
