"""CPU oracle of the MoE-layer forward: test infrastructure only.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  It shares no code with the HIP path.
"""
