"""CPU reference ("oracle") for per-rank context-parallel attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check and the bench's
CPU-baseline leg use it.  It shares no code with the HIP library and imports
nothing from it.

Everything is plain numpy in float64, written from the definitions in the
source pages:

* ``attention`` / ``attention_rows`` -- non-causal scaled dot-product
  attention returning O and the per-row log-sum-exp, with the full softmax
  row materialised ("Scaling AI inference across multiple GPUs using NVIDIA
  TensorRT with multi-device inference support", sections "Context
  parallelism" and "Ring Attention"; the scaled QK^T -> Softmax -> times V
  chain of the attention sample in "TensorRT multi-device attention
  inference in practice", step 1).
* ``merge`` -- combination of two partial (O, LSE) results over disjoint key
  sets, the algebra behind Ring Attention's online softmax (same page,
  section "Ring Attention").
* ``ulysses_pack`` / ``ulysses_unpack`` / ``alltoall`` -- the
  sequence<->head relayout around DeepSpeed Ulysses' two all-to-alls (same
  page, section "DeepSpeed Ulysses").
* ``rms_norm`` / ``qk_prologue`` / ``round_to_f16`` / ``round_to_bf16`` -- the
  QK-RMSNorm prologue of the attention sample (fp32 RMSNorm over head_dim,
  eps 1e-6, weight, cast to fp16, split score scale), with 16-bit rounding at
  the casts the page names ("TensorRT multi-device attention inference in
  practice", step 1).
* ``e4m3_to_f64`` -- decoding of the 8-bit float inputs of the fp8 attention
  path; the attention those inputs define is ``attention`` on the decoded
  values (fp8.py states the reading).

Pins: see tests/test_oracle.py (brute force, closed forms, invariants,
library special cases, merge algebra, relayout bijections, RMSNorm closed
forms and torch's rms_norm, 16-bit rounding ties).
"""
from .attention import attention, attention_rows
from .merge import merge
from .relayout import ulysses_pack, ulysses_unpack, alltoall, SEQ_TO_HEAD, HEAD_TO_SEQ
from .qk_norm import rms_norm, qk_prologue, round_to_f16, round_to_bf16
from .fp8 import e4m3_to_f64

__all__ = [
    "attention", "attention_rows", "merge",
    "ulysses_pack", "ulysses_unpack", "alltoall", "SEQ_TO_HEAD", "HEAD_TO_SEQ",
    "rms_norm", "qk_prologue", "round_to_f16", "round_to_bf16", "e4m3_to_f64",
]
