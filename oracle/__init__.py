"""CPU oracle of the randomized Hadamard rotation + symmetric quantisation.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's
CPU-baseline leg; the product package never imports it.
"""
