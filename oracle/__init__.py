"""Plain, slow fp64 CPU oracle of one quantized MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its Python binding) never imports, links or calls it, and this package
shares no code with that path: it decodes the packed weight formats itself,
routes, permutes and evaluates the FFNs in float64 with NumPy.

What it follows (page "Show HN: Menjalankan GLM 5.2 di komputer lambat"):
  * section "Fitur utama": a DeepSeek-V3-style sigmoid router with the
    bias-corrected group-limited selection ("noaux_tc"), renormalised weights
    times routed_scaling_factor, and a shared expert;
  * section "Fitur utama": batch-union MoE, where each unique expert of a batch
    is applied to every position routed to it (the permutation);
  * sections "Cara kerja eksekusi MoE" and "Fitur utama": int4 expert weights
    dequantised on use, and the per-row-scale int8 / packed int4 / packed int2
    formats of the quantisation kernels, and the integer-dot path with int8
    activations;
and page "NVIDIA stellt neues GLM-5.2 NVFP4 Modell vor", section "Technische
Details": the expert FFNs in 4-bit with one FP8 scale per 16 elements.

Parity pins: every function here is pinned by tests under tests/ that do not
re-use its own formula (closed forms, brute force, library routines, invariants).
The whole layer against an independent external implementation is "parity
unpinned": the pages print no worked example of the layer and their own
reference implementation and trained weights are not available.
"""
from .moe import (  # noqa: F401
    bf16_bits_to_f64, fp16_bits_to_f64, decode_e2m1, decode_e4m3fn,
    unpack_int4_codes, unpack_nvfp4_codes, dequant_int4, dequant_nvfp4,
    unpack_int2_codes, dequant_int4_row, dequant_int8_row, dequant_int2_row, ROW_FORMATS,
    A8_FORMATS, quantize_rows_int8, w4a8_ffn,
    RouterConfig, route, route_weights, route_margins, valid_under_perturbation,
    apply_top_p, valid_top_p,
    permute, swiglu_ffn, expert_ffn, layer, dense_layer, ExpertSource,
)
