"""Plain float64 CPU oracle for the certified KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, table
or constant generator with the HIP library under ``certified_kv_cache_amd``.

It is written from the WitCert pages ("WitCert: Sound Runtime Risk
Observability and Gating for KV-Cache Quantization", arXiv 2607.28699):

* ``dither``  -- the counter-hash dither regenerated at read time
  (m.montaan.com summary, Tier B paragraph) built on the published ``pcg``
  hash of Jarzynski and Olano, "Hash Functions for GPU Rendering", JCGT 9(3),
  2020.
* ``quant``   -- the write path: subtractively-dithered INT8, fp8 e4m3 raw
  cast, 2-bit asymmetric grouped, and the per-band residual-norm witness
  (summary, witness theorem paragraph; RULER results paragraph for fp8 and
  kivi-2bit).
* ``meter``   -- compressed decode attention, Tier A and Tier B per-token
  logit bounds, the total-variation aggregation, KV splits merged by
  log-sum-exp, block risks and the true TV it bounds.
* ``gate``    -- the fixed-point gate that selects blocks to page in.
* ``rope``    -- NeoX rotate-half RoPE and the frequency bands (Lemma 1).

Floating point is float64 except where the GPU must agree bit for bit (the
quantizers): there the oracle replays the stated float32 operation sequence
with numpy float32 scalar/array ops, each of which is correctly rounded.

Parity status of every function is listed in its docstring; functions whose
result has no pin against the pages or mathematics say "parity unpinned".
"""
