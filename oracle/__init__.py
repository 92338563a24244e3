"""CPU oracle for the LittleBit factored binary linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (``binary_rank_gemv_amd``) never imports it and
shares no code, table or helper with it.

Everything here is plain NumPy in float64 (plus ``fractions.Fraction`` for the
exact evaluator).  Each function cites the passage of the source pages it
follows; the pages are referred to by site and section:

* "explainx.ai explainer" -- the explainx.ai page "Samsung LittleBit: A 13B LLM
  Under 1 GB, and What the Paper Really Shows".
* "trueseeker fact-check" -- the trueseeker.com case page on the claim that
  LittleBit compressed Llama 2 13B from 26.06 GB to 0.84 GB.

Parity status of every function is listed in ``littlebit_oracle``'s module
docstring.
"""

from .littlebit_oracle import (  # noqa: F401
    sign_matrix,
    branch_weight,
    dense_weight,
    linear_forward,
    factored_forward,
    exact_forward,
    transposed_forward,
    rows_forward,
    bits_per_weight,
    rank_for_bpw,
    model_footprint_bytes,
)
from .dual_svid import (  # noqa: F401
    truncated_svd_factors,
    svid,
    dual_svid_branch,
    dual_svid_init,
    reconstruction_error,
    itq_rotation,
    itq_objective,
)
from .packing import (  # noqa: F401
    pack_factor,
    unpack_factor,
    packed_factor_bytes,
    sign_bits,
)
