"""Plain fp64 CPU oracle for streamed log-domain Sinkhorn (TEST INFRASTRUCTURE).

This package is the checker, not the product. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The HIP library under ``streaming_sinkhorn_amd/`` never imports,
links or calls anything here, and this package imports nothing from it.

Everything is written from the definitions on the page "FlashSinkhorn:
IO-Aware Entropic Optimal Transport on GPU" (arXiv 2602.03067):

* the squared-Euclidean cost is formed by the direct difference
  sum_k (x_ik - y_jk)^2, never by the norm expansion the GPU path uses;
* a Sinkhorn half-step is a plain log-sum-exp over the full dense row or
  column, with no tiling, streaming or online merging;
* the coupling, its marginals, P V, P^T U and the gradient are dense
  products of the materialised coupling;
* affine, cosine and label-augmented costs (``oracle.costs``, §3.1 "Scope
  of cost structure", §4.2) are dense matrices from their plain definitions;
* eps-scaling and the debiased Sinkhorn divergence (``oracle.divergence``)
  are the plain iteration at a decreasing eps and three dual values;
* the Hessian-vector product (``oracle.hvp``, §3.3 / App. F) is formed from
  the dense coupling, with the pseudoinverse by eigendecomposition or the
  damped Schur complement solved by textbook conjugate gradients.

Every function is pinned by the ``-m "not gpu"`` tests in ``tests/`` against
closed forms, textbook special cases and brute force (see each test's
docstring); none is "parity unpinned".
"""

from .sinkhorn import (  # noqa: F401
    sqnorms,
    cost_matrix,
    logsumexp,
    update_f,
    update_g,
    sinkhorn,
    sinkhorn_symmetric,
    plan,
    marginals,
    marginal_errors,
    apply_plan,
    apply_plan_t,
    barycentric,
    grad_x,
    dual_value,
    update_f_rows,
    update_g_cols,
    plan_rows,
    plan_cols,
)
from . import hvp  # noqa: F401,E402
from . import costs  # noqa: F401,E402
from . import divergence  # noqa: F401,E402
