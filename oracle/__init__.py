"""CPU oracle for NSA -- test infrastructure only (tests, smoke check, CPU baseline)."""
