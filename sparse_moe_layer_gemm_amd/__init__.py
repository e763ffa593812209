"""MI355X-native LatentMoE layer forward: HIP kernels behind a C ABI.

Importing the package loads nothing; `sparse_moe_layer_gemm_amd.binding`
loads the HIP library (liblatentmoe.so) on first use and fails loudly when it
is missing.
"""
