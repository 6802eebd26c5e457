"""CPU oracle for partitioned attention over a ring-buffer KV cache.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``partitioned_kv_cache_amd``) never imports, links or calls anything here and
fails loudly when its HIP library is missing.

Everything is plain NumPy in float64. Inputs arrive as float64 arrays holding
exactly the (bf16 or fp32) values the GPU reads, so the conversion is exact.
No code is shared with the HIP path; the two meet only at the seeded input
generator, which holds none of the method's arithmetic.

Sources (web pages about the method; cited by page title and section):

* "Reflex: Real-Time VLA Control through Streaming Inference" -- paper review
  (xllm-io blog): §3 Architecture (Eq. 1 partitioned attention, Eq. 2
  AdaRMSNorm, Prop. A.1 equivalence, component table), §5 Code analysis
  (ring-buffer initialisation, AdaRMSNorm module), §6 Experiments (Tables 4, 5, 7).
* "Reflex" reading notes (robotics-star): Method.
* "Reflex" summary (recoleta): Approach, Results.
* "OxyGen: Unified KV Cache Management for Vision-Language-Action Models under
  Multi-Task Parallelism" review (rainbus): core method, method details.

Modules
-------
attention  full-batch softmax attention over the chronological context (Eq. 1)
ring       the static ring buffer as a byte-level model (FIFO pin + slide)
adanorm    sinusoidal embedding, gamma MLP and AdaRMSNorm (Eq. 2)
stack      one layer of the denoising stack and the Euler update
decode     the shared-KV multi-reader (OxyGen) decode attention

Pin status of each function is listed in its docstring. Every function has
an external pin; the layer glue (a reading: the pages give none) is pinned
end to end against the same step written with torch's float64 operators.
"""

from . import attention, ring, adanorm, stack, decode  # noqa: F401
