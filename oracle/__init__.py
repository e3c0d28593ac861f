"""Plain CPU oracle for the routed MoE FFN layer.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
