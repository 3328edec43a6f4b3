"""MI355X ring all-reduce family: Python binding over the C-ABI library."""
