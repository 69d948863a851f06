"""CPU oracle for the INT4 2-bit-CSR SparseGEMV (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never does.
"""
from .i4s_oracle import (  # noqa: F401
    CANDIDATE_GROUP_SIZES, SLOT_TO_ELEMENT, OracleError, check_args, nm_mask,
    element_stream, group_scales, quantize, sse_units, choose_group_size,
    encode_vals, encode_codes, pack, decode, reconstruct, gemv, run,
    packed_nbytes, plain_csr_nbytes,
)
