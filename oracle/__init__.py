"""CPU oracle for the IM-Unpack integer GEMM path (test infrastructure only)."""
