"""CPU oracle for the TurboQuant hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 numpy implementation of what the GPU library computes,
written from the pages' description of the method:

* the coordinate law after a random rotation and the Lloyd-Max codebook on it
  (AiBoss overview "TurboQuant - Googleのベクトル量子化アルゴリズム",
  section "TurboQuantの技術原理"; ai-navigate-news Gemma 4 post, section
  "仕組み（技術的）", Algorithm 1);
* Algorithm 1 (TurboQuant_mse) and Algorithm 2 (TurboQuant_prod: Algorithm 1
  at b-1 bits plus sign(S r) of the residual) with dense bit packing and fp16
  norms / residual norms (same post, same section);
* decode attention with K through Algorithm 1 and V through Algorithm 2
  (same post, same section);
* inner-product search with top-k (AiBoss overview, section
  "TurboQuantの応用事例"; AIgent Lab explainer, section "視点3").

Only the test suite, the package's smoke check and the benchmark's CPU
baseline leg may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links it, and shares no code with
it: both sides receive the same seeded inputs and nothing else.
"""
from .codebook import coord_density, coord_tail, lloyd_max, gaussian_lloyd_max  # noqa: F401
from .quantizer import (  # noqa: F401
    fp16_rne_sat, encode_mse, decode_mse, encode_prod, decode_prod, pack_planes,
    unpack_planes, tile_records, mse_record, prod_record, parse_mse_record, parse_prod_record,
    inner_product_estimate, qjl_scale, code_margins, sign_margins, fp16_midpoint_margin,
)
from .attention import decode_attention  # noqa: F401
from .search import score_all, topk_desc, recall_at_k  # noqa: F401
