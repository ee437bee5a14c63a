"""Oracle package - TEST INFRASTRUCTURE ONLY (tests, smoke() and the CPU baseline of the
benchmark).  The product path never imports it."""
