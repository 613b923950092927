"""CPU oracle for the Sol-Attn forward pass: test infrastructure only.

Only tests, the smoke check and the bench's CPU-baseline leg may import it.
"""
