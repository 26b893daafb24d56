"""CPU oracle of the fused MoE expert layer. TEST INFRASTRUCTURE ONLY: the
test suite, the smoke check and the benchmark's CPU-baseline leg may use it;
the product package never imports it."""
