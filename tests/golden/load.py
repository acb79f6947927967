"""Reader for the key = value text fixtures in this folder."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            parts = val.split()
            if len(parts) == 1:
                v = parts[0]
                try:
                    out[key] = int(v)
                except ValueError:
                    try:
                        out[key] = float(v)
                    except ValueError:
                        out[key] = v
            else:
                try:
                    out[key] = [int(p) for p in parts]
                except ValueError:
                    out[key] = parts
    return out
