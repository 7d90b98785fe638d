"""Whole-workload parity figures collected during a test session.

The GPU parity tests append one line per compared tensor (max-abs and
mean-abs error over the whole workload); the test session prints them in its
terminal summary, where they survive output capture.
"""

LINES = []


def record(line: str) -> None:
    LINES.append(line)
