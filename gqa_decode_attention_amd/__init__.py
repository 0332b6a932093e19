"""MI355X (gfx950) grouped-query attention decode step.

Python face of the HIP library ``libgqa_decode.so`` (C ABI in
``include/gqa_decode.h``): ``append`` writes each sequence's new key/value at
slot ``lengths[b]`` of a fixed-capacity cache, ``attend`` runs length-masked
GQA attention over the cache, and ``step`` does both in one call; the
``_mapped`` calls take slot-indexed or paged caches and the ``_q8`` calls int8
caches with per-row scales; the ``_ex`` calls take any combination of a cache
map, int8 scales, rotary encoding (``Rope``) and softmax variants
(``Softmax``).  torch is
used for device memory and streams only.
"""
from ._lib import (  # noqa: F401
    BF16,
    EXPORTS,
    F32,
    FP8,
    I8,
    LIB_PATH,
    Desc,
    GqaError,
    MapT,
    OptsT,
    Rope,
    RopeT,
    Softmax,
    SoftmaxT,
    ScalesT,
    append,
    append_ex,
    append_q8,
    append_mapped,
    attend,
    attend_ex,
    attend_mapped,
    attend_q8,
    check_lengths,
    desc_for,
    get_plan,
    get_plan_ex,
    lib,
    make_desc,
    step,
    step_ex,
    step_mapped,
    step_q8,
    workspace_size,
    workspace_size_ex,
)
