"""Oracle for the attention forward and its gradients: plain, slow fp64 CPU code.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only callers. It shares no code with the HIP path.
"""

from .attention import attend_head, attend_head_grad, attention_grad_ref, attention_ref

__all__ = ["attend_head", "attention_ref", "attend_head_grad", "attention_grad_ref"]
