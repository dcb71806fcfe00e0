"""CPU oracle of the HARD-KV decode step -- TEST INFRASTRUCTURE ONLY.

Loaded by the tests, the smoke check and the benchmark's CPU baseline; never by
the product path.
"""
