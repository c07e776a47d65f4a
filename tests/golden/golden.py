"""Parser for the key: value fixtures in this folder (comments start with '#')."""
from pathlib import Path

HERE = Path(__file__).resolve().parent


def load(name: str) -> dict:
    out = {}
    for line in (HERE / name).read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, val = line.split(":", 1)
        out[key.strip()] = val.strip()
    return out


def hexbytes(s: str) -> bytes:
    return bytes(int(t, 16) for t in s.split())


def floats(s: str):
    return [float(t) for t in s.split()]
