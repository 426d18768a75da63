"""CPU oracle for the packed low-bit KV cache and decode attention.

Test infrastructure only: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product package. It shares no code with the HIP path.
"""
