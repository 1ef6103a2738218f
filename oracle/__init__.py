"""CPU oracle of the ISD step: test infrastructure, never the product path.

Plain, slow, obviously correct float64 numpy implementations of what the
HIP library computes, each module citing the passage of the pages it
follows. Only tests, the smoke check and the benchmark's CPU-baseline leg
import this package; the library and its binding never do, and the two
share no code. Modules:

  philox    Philox4x64-10 and the per-step uniforms
  attention paged KV write and causal GQA attention of the stride block
  accept    softmax, inverse CDF, the verify / resample / propose step
  lora      base projection and gated LoRA
  chain     the tokens-per-forward closed form and its two-state chain
  forward   RMSNorm, SwiGLU, bf16 rounding and a decoder block built
            from the modules above
"""

from . import accept, attention, chain, forward, lora, philox  # noqa: F401
