"""Figures the GPU parity tests collect for the end-of-run summary (printed by
conftest.pytest_terminal_summary)."""

# Top-k gap bands over the rows checked against float64 scores:
# band -> [rows, rows whose set equals the exact sort prefix]
GAP_STATS = {}
# free-form lines (worst error ratios and the like)
LINES = []
