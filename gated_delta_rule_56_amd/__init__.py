"""KDA (Kimi Delta Attention) on MI355X: HIP kernels behind a C ABI.

Importing the package loads nothing; ``gated_delta_rule_56_amd.kda`` loads
the native library on first use.
"""
__all__ = ["inputs", "kda"]
