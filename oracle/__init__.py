"""CPU oracle for group-wise low-bit weight quantization — TEST INFRASTRUCTURE ONLY.

A plain, slow, deliberately obvious numpy implementation of what the pages compute,
used to check the HIP library. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it; the product path (group_wise_bit_amd) never does,
and this package imports nothing from it.

Arithmetic conventions (stated once, used everywhere):
  * float32 ops are numpy float32 ufuncs: one IEEE-754 operation, round to nearest
    even, no fusion. Division is true division.
  * "round" on the pages is torch.round, i.e. round half to even: numpy.rint.
  * bfloat16 arithmetic is "compute in float32, round the result to bfloat16 (RNE)",
    which is how torch evaluates bf16 tensor ops; see _fp.bf16_round.
  * Reductions that the pages leave unordered (sums) are done in float64.

Modules:
  gptq   — 4-bit GPTQ symmetric uint4b8 and asymmetric int4 (page export_gptq_cpu.py)
  mxfp4  — OCP MXFP4: e2m1 codes, E8M0 block scale (page quantize_dflash_mxfp4.py)
  uintx  — torchao-style affine uint2..uint7 with planar bit shards (page uintx_quant.py)
  snr    — reconstruction SNR and relative error
  awq    — AWQ-style alpha search on MXFP4 (page quantize_dflash_mxfp4.py, search_scale)

Every function is pinned by tests/test_oracle_*.py against brute force, exact rational
arithmetic, closed forms, invariants and hand-derived worked examples.
"""
from . import gptq, mxfp4, uintx, snr, awq  # noqa: F401
