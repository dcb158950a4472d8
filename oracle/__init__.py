"""CPU oracle of the nested-weight speculative round -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package. The product path (nested_quantized_weights_amd) never
imports it.
"""
