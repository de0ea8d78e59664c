"""CPU oracle package: test infrastructure only (tests, smoke check, CPU baseline)."""
