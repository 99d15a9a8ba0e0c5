"""CPU oracle for the GRINQH decode GEMV: numpy (grinqh_oracle) and plain C.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
bench's CPU-baseline leg may import anything from this package.
"""
