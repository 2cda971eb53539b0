"""CPU oracle of the Wan-style video VAE decoder (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg use it.
"""
