"""NVFP4 W4A4 MoE GEMMs with Residual Activation Compensation on MI355X."""
