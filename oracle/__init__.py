"""CPU oracle for the CSA2 hot path. Test infrastructure only: the product path never imports it."""
