"""Plain, slow, fp64 CPU oracle of the TurboQuant KV-cache codec.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call, link
or execute anything in this package: only the test suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it. The
GPU library and this package share no code, tables, constants or helpers; the
only thing both sides consume is the seeded input arrays from ``synth``.

Every function follows a passage of the source pages, cited by page title and
section.  The pages (short names used throughout):

* [TurboQuant-es]  "Google presenta TurboQuant, un nuevo algoritmo de
  compresión ..." (7minutos.es news article).
* [TurboQuant-pl]  "TurboQuant: Jak rozwiązać największy problem pamięciowy AI
  za darmo" (securhub.pl blog).
* [FibQuant]       "FibQuant: Quantizzazione Vettoriale Universale per la
  Compressione della KV-Cache ad Accesso Casuale" (gist.science summary).
* [Ablation]       "Ablazione, Inferenza Statistica e Validazione per la
  Compressione della KV-Cache" (gist.science summary).
* [TurboESM]       "TurboESM: Quantizzazione Ultra-Efficiente a 3-Bit della KV
  Cache per i Modelli Linguistici delle Proteine ..." (gist.science summary).

Pins: every function here is pinned by a CPU test against closed forms,
textbook reductions, library routines the oracle does not itself use, or
brute force on tiny inputs (tests/test_oracle_*.py).  Parity unpinned: the
pages' model-quality numbers (cosine 0.96, needle recall, perplexity) are not
reproduced, since they need trained weights and datasets.
"""

from .codebook import (beta_coord_pdf, lloyd_max, codebook, distortion,
                       cell_moments)
from .rotation import (hadamard_sylvester, paley_hadamard_12, hadamard_matrix,
                       rotate, rotate_inverse, haar_rotation)
from .codec import (encode_mse, encode_prod, decode_mse, decode_prod,
                    estimate_ip, pack_codes, unpack_codes, pack_bits,
                    unpack_bits, EncodedMSE, EncodedProd, qjl_factor,
                    qjl_projection)
from .rope import rope_interleaved
from .attention import attention_from_codes, attention_materialized
from .search import inner_product_matrix, top_k
from .split import (outlier_permutation, effective_rate, encode_split_mse,
                    encode_split_prod, decode_split, estimate_split,
                    attention_split)
from .fibquant import (block_pdf, spiral_init, quadrature, nearest, block_mse,
                       lloyd, fibquant_codebook, encode_vq, decode_vq, pack_vq,
                       unpack_vq)

__all__ = [
    "beta_coord_pdf", "lloyd_max", "codebook", "distortion", "cell_moments",
    "hadamard_sylvester", "paley_hadamard_12", "hadamard_matrix", "rotate",
    "rotate_inverse", "haar_rotation", "encode_mse", "encode_prod",
    "decode_mse", "decode_prod", "estimate_ip", "pack_codes", "unpack_codes",
    "pack_bits", "unpack_bits", "EncodedMSE", "EncodedProd", "qjl_factor",
    "qjl_projection", "rope_interleaved", "attention_from_codes",
    "attention_materialized", "inner_product_matrix", "top_k", "block_pdf",
    "spiral_init", "quadrature", "nearest", "block_mse", "lloyd",
    "fibquant_codebook", "encode_vq", "decode_vq", "pack_vq", "unpack_vq",
    "outlier_permutation", "effective_rate", "encode_split_mse",
    "encode_split_prod", "decode_split", "estimate_split", "attention_split",
]
