"""Float64 CPU oracle for the GQA decode step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python binding)
never imports or calls it, and it imports nothing from them.
"""
from .oracle import (  # noqa: F401
    append,
    attend,
    attend_one,
    decode,
    kv_index,
    kv_rows,
    softmax_weights,
    step,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    decode_e4m3,
    encode_e4m3,
)
from .mapped import (  # noqa: F401
    append_mapped,
    append_q8_mapped,
    attend_q8_mapped,
    step_q8_mapped,
    attend_mapped,
    mapped_rows,
    slot_location,
    step_mapped,
    validate_slots,
    validate_table,
)
from .quant import (  # noqa: F401
    append_q8,
    attend_q8,
    code_format,
    dequantize,
    quantize_row,
    step_q8,
)
from .rope import (  # noqa: F401
    encode,
    rms_norm,
    rope_rotate,
    rotate_new,
    step_q8_rope,
    step_rope,
)
from .variants import (  # noqa: F401
    attend_variant_one,
    attend_variants,
    attended_slots,
    step_variants,
)
