"""fp64 CPU oracle for the ParaRNN Newton solve (test infrastructure only)."""
