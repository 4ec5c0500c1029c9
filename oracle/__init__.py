"""CPU oracle for block-sparse video attention (TEST INFRASTRUCTURE ONLY).

A plain, slow, fp64 numpy implementation of what the HIP library computes.
It exists to prove the library right; it is not a fallback.  Only the test
suite, the smoke check of the package entry file and the benchmark's CPU
baseline leg may import it.  It shares no code with the HIP path.

Sources (web pages; cited by page and section throughout):
  * SPADE review page, arXiv 2608.03335 ("SPADE: An Input-Adaptive Sparse
    Attention Engine for Fast Video Diffusion Models Inference").
  * Sliding Tile Attention verdict page, arXiv 2502.04507.
  * Sparse VideoGen verdict page, arXiv 2502.01776.
  * FG-Attn verdict page, arXiv 2509.16518.

Modules:
  geometry  - 3D tiling of the token grid, tile membership, windows
  layout    - tile-major permutation and its inverse
  select    - pooled means, tile scores, window / Top-K / Top-P masks
  sics      - SICS tile-coherence score and candidate blocking choice
  fine      - M x 1 fine-grained group mask
  attention - masked softmax attention (dense definition + block-sparse)
  fp8       - E4M3 quantization and the FP8 attention path
  profile   - online profiling selector (sampled-row MSE against full attention)
"""
from . import geometry, layout, select, sics, fine, attention, fp8, profile  # noqa: F401
