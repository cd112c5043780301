"""CPU oracle for the fused, chunked top-K KL distillation loss.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The HIP library and
its Python binding never import it, and it imports nothing from them.

See ``oracle/kl_oracle.py`` for what is computed and which passage each step
follows.
"""
from .kl_oracle import (  # noqa: F401
    to_f64,
    teacher_grid,
    student_log_softmax,
    kl_rows,
    kl_grad_logits,
    fused_kl_reference,
    rows_reference,
    reduction_weights,
)
from .teacher_oracle import teacher_logits, teacher_topk_reference  # noqa: F401
