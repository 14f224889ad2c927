"""Content-aware top-k block-sparse attention for AMD MI355X (gfx950).

The compute lives in libdsa.so (HIP kernels + C ABI, see include/dsa.h);
`binding` exposes its entry points to Python, `pipeline` chains them into
the prefill, decode and three-branch paths, `inputs` makes seeded synthetic
workloads and `configs` names them.
"""
from . import configs  # noqa: F401

__all__ = ["configs", "binding", "pipeline", "inputs", "metrics"]
