"""CPU oracle for the MXFP8 cast and grouped GEMM (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package. It shares no code with the HIP library and the library never calls it.
"""
from . import mx  # noqa: F401
