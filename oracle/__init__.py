"""CPU oracle for exact attention (test infrastructure only; see attn_oracle)."""
from .attn_oracle import (  # noqa: F401
    attention_oracle,
    attention_online_oracle,
    attention_oracle_rows,
    attention_rows,
    effective_scale,
    kv_length,
    valid_keys,
)
from .fp8_oracle import (  # noqa: F401
    attention_fp8_oracle,
    attention_fp8_oracle_rows,
    dequantize,
    e4m3_decode,
)
from .varlen_oracle import attention_varlen_oracle, seq_spans  # noqa: F401
from .softmax_oracle import softmax_rows, softmax_rows_four_pass  # noqa: F401
