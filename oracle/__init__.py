"""fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the bench's CPU-baseline leg may import, call, link or run anything in this
directory.  The product path (the HIP library and its Python binding) never
does, and this directory imports nothing from the product.
"""
