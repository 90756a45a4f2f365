"""Writes input_hashes.json: sha256 of the generated Q|K|V bf16 bytes per
workload (all heads; the 720p workload's head 0 only). It calls only the
seeded input generator. Run from the repository root:
    python tests/golden/make_input_hashes.py
"""
import hashlib
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import workloads as W  # noqa: E402

out = {}
for name, w in W.WORKLOADS.items():
    heads = [0] if name == "wan720" else None
    q, k, v = W.make_qkv(w, heads=heads)
    out[f"{name}:{'0' if heads else 'all'}"] = hashlib.sha256(q.tobytes() + k.tobytes() + v.tobytes()).hexdigest()
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_hashes.json")
with open(path, "w") as fh:
    json.dump({"_about": "sha256 of generated Q|K|V bf16 bytes, written by make_input_hashes.py",
               "hashes": out}, fh, indent=1)
print(json.dumps(out, indent=1))
