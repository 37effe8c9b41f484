"""CPU oracle of the fused adaLN path.  TEST INFRASTRUCTURE ONLY (tests, smoke check,
benchmark CPU baseline); the product path never imports this package."""
