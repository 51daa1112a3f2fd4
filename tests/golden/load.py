"""Reader for the small text fixtures in this folder."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def read_fixture(name):
    out = {"edges": [], "maximal": [], "not_maximal": [], "degree": {}}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            vals = [int(v) for v in vals]
            if key == "n":
                out["n"] = vals[0]
            elif key == "edge":
                out["edges"].append(tuple(vals))
            elif key in ("maximal", "not_maximal"):
                out[key].append(tuple(sorted(vals)))
            elif key == "degree":
                out["degree"][vals[0]] = vals[1]
            elif key == "maxdegree":
                out["maxdegree"] = vals[0]
    return out
