"""Reader for ``tests/golden/page_values.txt`` (values stated on the pages)."""
import os

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_values.txt")


def page_values() -> dict:
    out = {}
    with open(_PATH) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out[key] = float(val) if "." in val else int(val)
    return out
