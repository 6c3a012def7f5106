"""fp64 CPU oracle for the group-scaled binary / ternary matrix product.

Test infrastructure only (tests, smoke check, benchmark CPU baseline)."""
