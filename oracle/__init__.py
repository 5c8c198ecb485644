"""CPU oracle for replay attention: test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It is plain float64 numpy written from the definition of attention and shares
no code with the HIP library.
"""
from .attention import (  # noqa: F401
    backward,
    capture_pages,
    delta,
    forward,
    forward_parts,
    gather_pages,
    lse_merge,
    lse_merge_bf16_numerator,
    round_bf16,
    shard_token_bounds,
)
