"""Loader for the text fixtures under tests/golden/ (``key = <json>`` lines,
``#`` comments carry the citation of the page the values were printed on)."""
import json
import os

_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(_DIR, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            out[k.strip()] = json.loads(v.strip())
    return out
