"""CPU oracle for the grouped 4-bit expert GEMM — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product (the HIP library and its Python binding) never calls
it, and it shares no code with the product: it is a plain, slow, fp64 numpy
restatement of what the method computes, written so that each step can be
checked against the source pages by eye.

Sources (web pages about the `grouped-nf4-gemm` package, cited by title and
section):

* "grouped-nf4-gemm 0.33.1" (PyPI project page), opening description: one launch
  computes the expert GEMM for every routed expert straight from 4-bit codes; each
  code goes through a 16-value table, is multiplied by its block scale, products
  are summed in fp32 and the result is rounded to bf16. NF4 follows the
  bitsandbytes 4-bit layout; MXFP4 is OCP e2m1 codes with e8m0 block scales.
* "grouped-nf4-gemm releases", v0.2.6 section "The patch point": the result is
  the one of the per-expert loop that the kernel replaces — activation rows
  sorted by expert, `sizes[e]` rows for expert e, one matmul per expert.
* "grouped-nf4-gemm 0.33.1", section "Try it on CPU right now", blocks 1 and 2:
  packer shapes, round-trip errors of about 0.09 (NF4) and 0.12 (MXFP4), and
  that re-packing a decoded NF4 weight gives the same bytes.
* "grouped-nf4-gemm capability index" (index.json), `system_manifest.owns`: the
  package owns the input gradient of the grouped GEMM, dX = dY . W, computed on
  the same packed bytes.
* "grouped-nf4-gemm releases", v0.2.5 section (arena_experts), and the capability
  index's `entrypoints` (`swiglu_rows`): the fused expert block, gate_up -> SwiGLU
  -> down (oracle.block, with its readings stated there).
* The capability index's `entrypoints` (`router_epilogue`, `combine_rows`) and
  releases v0.2.6 "The patch point": the routing sort in front of the grouped
  GEMM and the top-k combine after it (oracle.route).
* "grouped-nf4-gemm releases", v0.2.4 section: the trainable low-rank delta
  B(Ax) composed with the frozen 4-bit projection at the pre-activation point
  (oracle.lora).
* "bw24 releases, v0.9.0", "Changes since v0.8.0": the W4A8 variant, e4m3
  activations times native e2m1 weights in one block-scaled matrix instruction
  (oracle.w4a8, with its readings of the activation scaling stated there).

Two public specifications that the pages rely on but do not print supply the
value tables: the NF4 data type (QLoRA, Dettmers et al. 2023, appendix E) and
the OCP Microscaling Formats (MX) v1.0 specification (e2m1 element, e8m0 scale).

`PARITY` below says what pins each function (tests/test_oracle_*.py).
"""
from .codebooks import (NF4_TABLE_F32, NF4_TABLE_BITS, nf4_table_closed_form,
                        e2m1_value, E2M1_TABLE, e8m0_value)
from .pack import (quantize_pack_nf4, dequant_nf4, unpack_nf4_codes, pack_nf4_codes,
                   quantize_pack_mxfp4, dequant_mxfp4, unpack_mxfp4_codes,
                   pack_mxfp4_codes, nf4_w32, mxfp4_w32, bf16_rne_bits, fp16_rne_bits)
from .grouped import (offsets, grouped_ref, loop_ref, dgrad_ref,
                      sampled_fwd_ref, sampled_dgrad_ref, brute_force_ref,
                      brute_force_dgrad)
from .block import (silu, swiglu_ref, bf16_rne_from_f64, expert_block_ref,
                    sampled_block_ref, brute_force_block)
from .route import route_sort_ref, gather_ref, combine_ref, brute_force_route
from .lora import lora_delta_ref, lora_forward_ref, lora_backward_ref, brute_force_lora
from .w4a8 import (E4M3_TABLE, e4m3_value, e4m3_round, mxfp8_scale_bytes, quantize_mxfp8,
                   dequant_mxfp8, w4a8_grouped_ref, sampled_w4a8_ref, brute_force_w4a8)

PARITY = {
    "NF4_TABLE_F32": "pinned: published decimal values and closed-form quantiles",
    "e2m1_value / E2M1_TABLE": "pinned: OCP value fixture tests/golden/e2m1_ocp.txt",
    "e8m0_value": "pinned: math.ldexp over all 256 bytes, NaN at 255",
    "quantize_pack_nf4": "pinned: page shapes, rel-err ~0.09, idempotence, "
                         "brute-force nearest code",
    "quantize_pack_mxfp4": "pinned: page shapes, rel-err ~0.12, brute-force nearest",
    "nibble order": "parity unpinned against external bytes (no released bytes "
                    "are available); pinned only by the stated convention",
    "grouped_ref": "pinned: pure-Python brute force, exact integer cases, loop_ref",
    "dgrad_ref": "pinned: adjoint identity with grouped_ref, pure-Python brute force",
    "silu / swiglu_ref": "pinned: closed forms (silu(0), silu(ln 3), the odd-part "
                         "identity silu(x) - silu(-x) = x), interleaved pair order",
    "bf16_rne_from_f64": "pinned: equals the bit-pattern rounding on fp32 inputs, "
                         "a double-rounding case, subnormals, ties to even",
    "expert_block_ref": "pinned: pure-Python brute force (math.fsum, math.exp), "
                        "zero up rows give zero output, exact integer case",
    "route_sort_ref": "pinned: pure-Python brute force, permutation and sortedness "
                      "invariants, the order loop_ref meets rows in",
    "combine_ref": "pinned: one-hot weights give the routed row exactly, "
                   "linearity in the weights, dropped slots",
    "E4M3_TABLE / e4m3_round": "pinned: torch float8_e4m3fn values and conversion "
                               "(every tie midpoint included), saturation at 448",
    "quantize_mxfp8": "pinned: OCP scale rule on hand-worked blocks, block maximum in "
                      "[256, 512), half-step error bound",
    "w4a8_grouped_ref": "pinned: pure-Python brute force (exhaustive nearest e4m3 "
                        "search, math.fsum), closeness to the bf16 product",
    "lora_forward_ref / lora_backward_ref": "pinned: torch fp64 autograd of the same "
                        "forward (independent derivatives), pure-Python brute force, "
                        "s = 0 reduction, linearity in s",
}

__all__ = [n for n in dir() if not n.startswith("_")]
