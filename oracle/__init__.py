"""CPU oracle for paged-KV attention forward — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct float64 NumPy code that states what the
GPU library must compute.  Only the test-suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product
path (the HIP library and its Python binding) never does, and this package
imports nothing from the product.

Sources (the five pages on paged-KV attention):

* "Triton-TLE rewrite of Tencent HPC-Ops Attention" (flagos.csdn.net),
  §1.2 (prefill pipeline: QK, causal mask, fp32 online softmax, PV,
  epilogue; paged addressing through the block table; block-mask tile
  skipping; dynamic decode Assign / Split-K / Combine) and §3.3 (merge of
  raw online-softmax states).
* "Chunked Prefill kernel optimisation: Triton hybrid attention"
  (xdnf.cn), mask specialisation: decode rows see their whole history,
  a prefill chunk is causal within itself and unmasked over its history.
* "HiLS-Attention sliding-window forward" (flagos.csdn.net), §3 stage 1:
  LSE in natural log, output layout (B, Hq, Lq, Dv), expand_to_chunk and
  the landmark rule (j + 1) mod C != 0.
* "vLLM Triton Attention Backend Deep Dive" (papercache), §3: Q blocks
  group all query heads of one KV head.

Modules
-------
fp8        OCP E4M3FN decoder (table built from the format definition).
attention  the definition: gather pages, mask, softmax(QK^T*scale)V, ln-LSE.
brute      pure-Python triple loops on dense (unpaged) K/V, tiny inputs.
split      attention restricted to a key range + the LSE-weighted combine.
taskmap    integer reference of the Assign work split.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force and ``torch`` library routines.
Parity status per function is listed in each module header.
"""
