"""rope_fp8_quant_amd - placeholder; the binding is added with the HIP library."""
