"""fp64 CPU oracle (test infrastructure only; see kl_oracle and topk_cache)."""
from .kl_oracle import as_f64, teacher_distribution, student_lse, fused_kl, fused_kl_rows  # noqa: F401
from .topk_cache import topk_cache, teacher_logits  # noqa: F401
