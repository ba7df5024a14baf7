"""fp64 CPU oracle for scaled dot-product attention.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
definition the fused HIP kernels are checked against. Only the tests, the
smoke check (``__graft_entry__.smoke``) and the benchmark's CPU-baseline leg
may import it; the product path (``scaled_dot_product_18_amd``) never does and
never falls back to it. It shares no code with the HIP path; the only module
both sides use is the seeded input generator ``sdpa_inputs``, which holds no
attention arithmetic.

Pins (tests marked "not gpu" that tie the oracle to something other than
itself): closed forms (one key, two keys with weights exactly 1/4 and 3/4,
causal first row), invariants (rows sum to one, equal keys give the mean of
V, causal last row equals the unmasked one, GQA equals MHA on repeated KV
heads, key shift, affine V, key permutation), brute force at 50 digits on
tiny inputs, torch's own fp64 CPU attention routine as an independent
library special case, hand-derived fixtures under tests/golden/, and the
E4M3 decoder checked exhaustively against torch.float8_e4m3fn; the
dequantiser (code times per-tensor descale) pinned by the amax element
mapping back to the amax and every element of a quantised tensor
round-tripping within half an E4M3 step; likewise the E5M2 decoder of the
fp8 backward pass's gradients, exhaustively against torch.float8_e5m2.

The gradients (backward.py) are pinned by central finite differences of the
forward oracle, closed forms (zero query, equal value rows, a single key), the
GQA head-sum identity and torch's fp64 autograd of its CPU attention.
"""

from .attention import attention, attention_rows, attention_sampled  # noqa: F401
from .backward import attention_backward  # noqa: F401
from . import e4m3  # noqa: F401
from . import e5m2  # noqa: F401
