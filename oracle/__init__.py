"""CPU oracle for the FlashDecoder per-latent-frame decode step.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark import this package.  The HIP decode path never calls it, and
it imports nothing from that path.

See `oracle.decoder` for the definition followed and the sources cited.
"""
from .decoder import (  # noqa: F401
    patchify, unpatchify, linear, layer_norm, rms_norm, kv_norm, gelu, attention,
    rope_split, rope_angles, apply_rope, token_rope_angles, split_qkv,
    subframe_rope_angles, subframe_tokens, spatial_upsample,
    StreamingDecoder, bruteforce_decode, as_f64_weights, host_threads,
)
