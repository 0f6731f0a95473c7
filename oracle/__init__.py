"""CPU oracle for the prefill attention-unit path (fp64 numpy, slow on purpose).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here.  The
product path (``prefill_causal_attention_amd``) never imports it, and this
package imports nothing from the product path: the two share no kernels,
helpers, tables or constants.  Inputs come from ``workloads`` (random draws
only).

Sources.  The method is taken from three web pages; each function cites the
page and section it follows:
  * [P1] "Prefill decoder-layer attention data flow" (hncyxsy.com/news/270449)
  * [P2] "Prefill vs decode tuning notes" (hncyxsy.com/news/227904)
  * [P3] "Decoding LLM inference latency: prefill bottlenecks"
         (lnwmold.com/news/496245)
The OCP 8-bit floating point specification (E4M3 encoding) defines the fp8
codec, which the pages only name.

What is computed is the plain definition: attention with a materialised score
matrix, an explicit additive -inf causal mask and a two-pass softmax, in fp64.
The pages' blockwise online-softmax form is also written out
(``attention.online_softmax_attention``) and pinned to equal the plain form.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
values the pages print, closed forms, invariants or brute force; nothing is
"parity unpinned".
"""
from . import bf16, fp8, attention, projection, kvcache  # noqa: F401
from . import fp8_attention  # noqa: F401
