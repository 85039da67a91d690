"""Oracle for the attention forward: a plain, slow fp64 CPU implementation.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only callers. It shares no code with the HIP path.
"""

from .attention import attend_head, attention_ref

__all__ = ["attend_head", "attention_ref"]
