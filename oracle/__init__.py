"""CPU oracle for the TurboQuant KV-cache quantizer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``kv_cache_vector_amd``); the two meet only through the seeded input
generator in ``synth`` and through the arrays the tests hand to both.

Plain, slow, obviously correct: float64 numpy, one step per line of the
method, no blocking, no fusion, no shortcut the pages do not state.

Sources (cited by short tag in every docstring):

[Scratch]  "TurboQuant From Scratch on Real KV Tensors -- What 3 Bits Actually
           Cost, and Why the Forks Beat the Paper's Layout"
           (www.sotaaz.com/post/turboquant-scratch-en).  Sections used:
           §2 "The Algorithm in 60 Lines", §3 "Sanity Check", §6 "Finding 3:
           Norm Correction", §7 "Finding 4: Block-32".
[README]   "turboquant-pytorch" README (github, ringlorn/turboquant-pytorch):
           the two-stage description, the combined inner-product estimator,
           the tables "MSE Distortion (d=128, 1000 random unit vectors)" and
           "Inner Product Accuracy (d=128, 2000 random vector pairs)".
[Fork]     "TurboQuant KV Cache Quantization (Experimental)"
           (llama.cpp-turboquant docs/turboquant.md): "How it works",
           "GGML Types", "KV Cache Memory", "Fused tile path: K and V decoded
           inside attention".  ``blocks.py`` holds its 32-value record format.
[Blog]     "TurboQuant: 3-Bit Compression with Zero Overhead"
           (cneuralnets.xyz/blog/turboquant): "Part 2: Quantized
           Johnson-Lindenstrauss", "Part 3: TurboQuant Synthesis".

Every function here is pinned by ``tests/test_oracle_*.py`` against values
the pages print, closed forms, invariants or brute force.
"""
from .codebook import Codebook, lloyd_max_gaussian, gaussian_distortion, lloyd_max_beta, beta_distortion  # noqa: F401
from .quantizer import (  # noqa: F401
    fwht, hadamard_matrix, index_to_code, code_to_index, pack_codes, unpack_codes, pack_sign_bits,
    unpack_sign_bits, encode_indices, quantize, dequantize, qjl_scores, QJL_CONST,
)
from .attention import decode_attention, multi_attention  # noqa: F401
from .blocks import to_blocks, from_blocks, dequantize_blocks, record_bytes  # noqa: F401
