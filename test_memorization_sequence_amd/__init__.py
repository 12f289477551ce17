"""Test-time memory (ATLAS / Titans long-term memory) for MI355X: chunked
Omega-rule update with Titans momentum and decay, plus retrieval, as
hand-written HIP kernels behind the C ABI in include/atlas_mem.h."""
from .configs import WORKLOADS, ORDER, Workload  # noqa: F401
