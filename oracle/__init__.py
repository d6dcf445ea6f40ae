"""CPU oracle for the DFlash block-drafter proposal pass (test infrastructure
only: imported by tests, the smoke check and the benchmark's CPU baseline)."""
