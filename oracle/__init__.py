"""CPU oracle for block-sparse global attention with pooled and drift selection.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The HIP path never
routes through it, and it shares no code with the HIP path: no kernels,
headers, helpers, tables, pre- or post-processing. Inputs come from the seeded
generators in ``workloads`` (which hold no arithmetic of the method).

Everything is plain numpy in float64 on the exact input values (bf16 inputs are
widened exactly). Each function follows one step of the method in the order
the pages give it, without blocking, fusion or reordering.

Sources (pages, by title):
  * "ReSS: Residual-Restoring Sparse Attention for 3D Vision Transformers"
    (thelatestinai.com, 2609.35593) - abstract, Figs. 1-3, Tables 1, 2, S3, S5.
  * "VASC: Value-Aware Sparse Attention with Cross-Layer Memory for Efficient
    3D Reconstruction" (paperlayer.ai summary, 2610.01013v1) - sections 3,
    4.1-4.3, A.1-A.5 (value-aware selection and pair memory: oracle/vasc.py).

Parity status: every function below is pinned by tests/test_oracle_*.py
(closed forms, brute force, exhaustive search, hand-derived golden fixtures).
Equivalence with the published ReSS / SparseVGGT / VASC code is parity
unpinned: no code or step-level numbers of theirs exist on the pages.
"""
from .reference import *  # noqa: F401,F403
from .vasc import *  # noqa: F401,F403
