"""CPU oracle (test infrastructure; never imported by the product path)."""
from .qgemv_oracle import (  # noqa: F401
    abs_product_sum,
    bf16_bits_to_f64,
    check_close,
    dequantize,
    fp16_bits_to_f64,
    qgemv_add_reference,
    qgemv_reference,
    residual_f64,
    tolerance,
    unpack_codes,
)
