"""CPU oracle of the fixed-pool, three-wave MoE layer.

Test infrastructure only: imported by tests/, by the package smoke check and
by the CPU-baseline leg of bench.py; never by the product path.
"""
