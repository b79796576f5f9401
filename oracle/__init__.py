"""CPU oracle for 4-bit block-quantized dequantization and GEMV.

Test infrastructure only: the tests, the smoke check and the benchmark's CPU
baseline may import this package; the library and its Python binding never do.
"""
