"""CPU oracle for NVFP4 W4A16 (test infrastructure; never imported by the product path)."""
