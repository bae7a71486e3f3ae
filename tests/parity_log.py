"""Record of every GPU-vs-oracle comparison made in a test session.

Each test module's comparison helper calls record(); the session-end hook in
conftest.py prints the worst relative L2 and max-abs errors per group, so a
quiet (-q) run still reports the error magnitudes, not only pass counts.
"""
RECORDS = []


def record(what: str, rel: float, mx: float) -> None:
    RECORDS.append((what, float(rel), float(mx)))


def group_of(what: str) -> str:
    """Group key of a comparison label: the workload name when the label
    starts with one (c1..c5), else the first word."""
    head = what.split()[0] if what.split() else what
    return head
