"""The attention parity bar shared by every GPU test and smoke(); defined with the oracle
(``oracle/tolerance.py``) so that bench.py's CPU leg applies the same bar."""
from oracle.tolerance import BAR_TEXT, MANTISSA_BITS, TOL, bar, check, excess, half_ulp, summary  # noqa: F401
