"""Engram oracle: a plain CPU implementation used to check the HIP library.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
benchmark's CPU-baseline leg may import it. It shares no code with the
library under gram_hashed_embedding_amd/ and never calls it.
"""
