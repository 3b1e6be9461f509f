"""Scalar CPU oracle of the FlashLoop packed-KV codec -- test infrastructure only.

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP implementation.
"""
