"""CPU oracle of the local MoE forward pass -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The GPU library never does, and nothing here imports the GPU library.
"""
