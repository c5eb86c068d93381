"""CPU oracle for the MegaMoE expert pipeline.  Test infrastructure only."""
