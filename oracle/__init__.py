"""CPU oracle for one decode step of paged attention over a packed-FP8 KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, tables or
helpers with the HIP library under ``paged_fp8_kv_amd/``.

Every function here is written from the definitions on the source pages and is
deliberately slow and plain: numpy in float64 for all floating-point work,
integer arithmetic for all indexing, no blocking or fusion.

Sources (cited by page title and section throughout):
  * "GPT-OSS-120B giga-kernel decode" (AWS Neuron vllm-neuron design doc):
    sections "Kernel contract", "KV-cache layout (per-buffer, HMA-preserving)",
    "DI wiring (NIXL)", "KV budget (no cap)".
  * "determine_available_memory design" (AWS Neuron vllm-neuron design doc).

Modules:
  fp8_e4m3   OCP E4M3 codec (decode table, round-to-nearest-even saturating encode)
  layout     byte layout of one shared KV buffer, packed-K and plain-V addressing
  control    layer-invariant attention control (trimmed SWA table, positions,
             the two KV-update indices)
  update     quantize-and-scatter of the new token's K/V (K optionally rotated)
  rope       the rotary embedding of the new query and key (half-split pairing)
  attention  paged decode attention in float64 (plus a dense brute-force twin)
  step       the alternating SWA/full layer schedule over shared buffers
  budget     the KV-cache byte and block budget of a device (host policy)

Parity status: every function is pinned by a ``-m "not gpu"`` test (see the
test modules named ``tests/test_oracle_*.py``); none is "parity unpinned".
"""
