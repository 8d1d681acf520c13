import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Decision-parity summary of the GPU tests that named their layer: heads
    checked per route, ties (within 1e-6 of a threshold; counted, not failed)
    and heads exempt from the list comparison (PE cut inside the fixed-point
    error band)."""
    try:
        from tests import parity
    except Exception:
        return
    if not parity.REPORTS:
        return
    tr = terminalreporter
    tr.write_sep("-", "decision parity (bit-exact against the oracle on the GPU's float32 scores)")
    for name, r in parity.REPORTS:
        tr.write_line(f"{name}: tau {r['tau']:g} alpha {r['alpha']:g} gamma {r['gamma']:g}"
                      f"{' flags ' + str(r['flags']) if r['flags'] else ''}"
                      f"{' min_blocks ' + str(r['min_blocks']) if r['min_blocks'] else ''}: "
                      f"checked {r['heads_checked']} (VS {r['vs_heads']}, PE {r['pe_heads']}, dense {r['dense_heads']}); "
                      f"ties route {r['route_ties']} VS {r['vs_ties']} PE {r['pe_ties']}; "
                      f"exempt PE {r['pe_exempt']} VS {r['vs_exempt']}")
