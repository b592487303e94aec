"""Reader for the cited page numbers in page_numbers.txt."""
import os

_HERE = os.path.dirname(os.path.abspath(__file__))


def page_numbers(name: str = "page_numbers.txt") -> dict:
    out = {}
    with open(os.path.join(_HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split()
            out[k] = float(v)
    return out
