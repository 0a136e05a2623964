"""CPU oracle for absorbed MLA decode attention.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, float64 statement
of what the GPU path computes.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product
library (``mla_latent_kv_absorbed_amd``) never imports, links or calls it,
and it imports nothing from the product library.

Sources (all on the page "Kimi K3 decode: DP16 vs DP2 x DCP8" and the page
"resident VRAM accounting"):

* One latent row per token and layer: ``kv_lora_rank + qk_rope_head_dim``
  elements, stored once with no head dimension (VRAM page, section
  "KV ledger", MLA bullet; section "cell_size", MLA pool shape).
* ``kv_b_proj`` is absorbed into ``w_kc`` / ``w_vc`` (DP16-vs-DP2 page,
  section on the weight AllGather), and ``w_kc`` maps the 128-wide no-RoPE
  query to the 512-wide latent (same page, VRAM-ledger section, replicated
  Q projection bullet), so scores are taken in the latent space and the
  values are the latent itself.
* All query heads share the single latent KV head: the DP2 kernel is an MQA
  kernel (DP16-vs-DP2 page, section "MLA").
* Decode verifies 5 tokens per request per step (same page, introduction).
* DCP shard r holds the token slots p with p % 8 == r (same page, section
  "problem: how to split 16 GPUs").
* Partial results are (O, LSE) pairs merged by log-sum-exp (same page,
  section "MLA", the dcp_exchange / dcp_lse_combine bullets).

The formula itself is never written on the pages; the readings taken where
they are silent are listed in the module docstring of ``mla_ref``.

``fp4_ref`` defines the FP4 KV rows (e2m1 codes with one power-of-two
scale per 16 elements; VRAM page, "KV ledger" and "cell_size" sections) and
their quantiser; ``mxfp8_ref`` the MXFP8 rows (e4m3fn codes with one
power-of-two scale per 32 elements; "cell_size" section).  ``prepare_ref``
is the oracle of the step before attention (Q absorption, RoPE, KV
append), ``project_ref`` that of the step after it (the LSE merge followed
by the w_vc up-projection); their readings are in their own module
docstrings.
"""

from .mla_ref import (  # noqa: F401
    D_C,
    D_R,
    D_K,
    D_V,
    E4M3FN_TABLE,
    e4m3fn_decode_table,
    bf16_bits_to_f64,
    visible_positions,
    local_index,
    gather_slots,
    dequant_rows,
    query_rows,
    scores,
    softmax_reduce,
    mla_decode_ref,
    lse_combine_ref,
)
from .prepare_ref import (  # noqa: F401
    e4m3fn_encode,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    rope_f32,
    q_absorb_ref,
    q_rope_ref,
    latent_rows_ref,
    fp8_quantise_rows,
    kv_append_ref,
    mla_prepare_ref,
)
from .fp4_ref import (  # noqa: F401
    E2M1_TABLE,
    e2m1_decode_table,
    e2m1_encode,
    decode_fp4_rows,
    block_exponent_of,
    fp4_quantise_rows,
)
from .mxfp8_ref import (  # noqa: F401
    decode_mxfp8_rows,
    mxfp8_quantise_rows,
)
from .project_ref import (  # noqa: F401
    vc_project_ref,
    lse_combine_project_ref,
)
