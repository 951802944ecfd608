"""Readers of the text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def one_stage_cases():
    """(W, numel, hidden, dtype, fully_connected, expected, note) per line."""
    rows = []
    with open(os.path.join(GOLDEN, "one_stage_cases.txt")) as f:
        for line in f:
            body, _, note = line.partition("#")
            fields = body.split()
            if not fields:
                continue
            W, numel, hidden, dtype, fc, exp = (int(x) for x in fields)
            rows.append((W, numel, hidden, dtype, fc, exp, note.strip()))
    return rows
