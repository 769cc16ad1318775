"""fp64 CPU oracle (test infrastructure only; see kl_oracle)."""
from .kl_oracle import as_f64, teacher_distribution, student_lse, fused_kl, fused_kl_rows  # noqa: F401
