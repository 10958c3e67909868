"""fp64 CPU oracle — test infrastructure only (tests, smoke check, CPU baseline)."""
