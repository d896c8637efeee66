"""CPU oracle for D = A*B + C (test infrastructure only; see oracle.h)."""
