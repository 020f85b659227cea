"""Writes inputs_first8.txt: the first eight values of each seeded tensor of
two workloads, computed here one value at a time with Python integers and the
math module from the generator's published definition (splitmix64 of Steele,
Lea and Flood; the Box-Muller transform; round-to-nearest-even to fp32 and
bf16).  It imports nothing from the library, so the stored values pin the
vectorised generator that both the GPU path's callers and the oracle use.

    python tests/golden/make_inputs_golden.py
"""
import math
import os
import struct

MASK = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def bf16(x):
    u = struct.unpack("<I", struct.pack("<f", x))[0]
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return struct.unpack("<f", struct.pack("<I", u))[0]


def first_values(seed, tensor_id, count, dtype, scale):
    key = mix(seed * 16 + tensor_id)
    out = []
    for m in range((count + 1) // 2):
        x1 = mix((key + (2 * m + 1) * GAMMA) & MASK)
        x2 = mix((key + (2 * m + 2) * GAMMA) & MASK)
        u1 = (x1 >> 11) * 2.0 ** -53
        u2 = (x2 >> 11) * 2.0 ** -53
        r = math.sqrt(-2.0 * math.log1p(-u1))
        for z in (r * math.cos(2.0 * math.pi * u2), r * math.sin(2.0 * math.pi * u2)):
            v = f32(z)
            if scale is not None:
                v = f32(v * f32(scale))  # fp32 product, correctly rounded
            out.append(bf16(v) if dtype == "bf16" else v)
    return out[:count]


# workload, seed, dtype, scale of Q/K/V (dO is never scaled)
CASES = [
    ("single-head-n1k-ring-p4", 1001, "f32", None),
    ("llama7b-n32k-balanced-p8-fwd", 1002, "bf16", 1.0 / math.sqrt(128)),
    ("llama7b-n32k-balanced-p8", 1003, "bf16", 1.0 / math.sqrt(128)),
    ("llama7b-n131k-striped-p16-rank0", 1004, "bf16", None),
    ("gqa-32-8-n256k-balanced-p32", 1005, "bf16", None),
]
NAMES = ("q", "k", "v", "do")


def main():
    lines = ["# First eight values (logical [batch, token, head, head_dim] order) of each",
             "# seeded tensor; written by make_inputs_golden.py.",
             "# workload  seed  dtype  tensor  values (float32, repr)"]
    for wl, seed, dtype, scale in CASES:
        for tid, name in enumerate(NAMES):
            vals = first_values(seed, tid, 8, dtype, scale if name != "do" else None)
            lines.append(f"{wl} {seed} {dtype} {name} " + " ".join(repr(v) for v in vals))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "inputs_first8.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
