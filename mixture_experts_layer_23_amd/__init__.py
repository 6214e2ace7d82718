"""Local mixture-of-experts forward pass for AMD Instinct MI355X (gfx950).

``mixture_experts_layer_23_amd.moe`` is the thin Python binding of the C-ABI HIP library
``librudnn_moe.so`` (route, dispatch, SwiGLU experts, combine, full forward);
``mixture_experts_layer_23_amd.inputs`` draws the seeded synthetic workloads.  Importing the
package loads neither.
"""
