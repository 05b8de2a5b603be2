"""Fuzz of adam_state_load with mutated checkpoint streams (run by
tests/test_sanitizers.py in a process with the sanitizer runtimes preloaded,
against a sanitized host-only build of the library given as argv[1]).

Every mutated stream must be refused with ADAM_EINVAL -- or, if it is still
well formed, fail only at the first device call (no GPU here) -- and no
access may leave the buffer: AddressSanitizer aborts the process on one."""
import ctypes
import os
import random
import struct
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TESTS = os.path.dirname(HERE)
sys.path[:0] = [os.path.dirname(TESTS), TESTS]

import memory_efficient_adam_amd._binding as B  # noqa: E402

B._LIB_PATH = sys.argv[1]
import test_abi_host as T  # noqa: E402  (stream builder and checksum)

lib = B.library()
rng = random.Random(int(sys.argv[2]) if len(sys.argv) > 2 else 1234)
bases = [T._serialized([5000, 17], storage=s, options=o) for s in (1, 2, 3) for o in (0, 1)]
bases += [T._serialized([1]), T._serialized([0, 0, 2048]), T._serialized([4097], storage=3, options=1)]
EXTREME = [0, 1, 15, 16, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFF, 2 ** 32, 2 ** 62, 2 ** 63, 2 ** 64 - 1]


def rehash(b):
    b = bytearray(b)
    if len(b) >= 8:
        b[-8:] = struct.pack("<Q", T._stream_hash(bytes(b[:-8])))
    return bytes(b)


def mutate(b):
    b = bytearray(b)
    kind = rng.randrange(5)
    if kind == 0 and b:                      # flip a few bits
        for _ in range(rng.randint(1, 8)):
            i = rng.randrange(len(b))
            b[i] ^= 1 << rng.randrange(8)
    elif kind == 1 and len(b) >= 8:          # an extreme value in a 4- or 8-byte field
        w = rng.choice((4, 8))
        i = rng.randrange(0, len(b) - w + 1) // w * w
        b[i:i + w] = (rng.choice(EXTREME) & (2 ** (8 * w) - 1)).to_bytes(w, "little")
    elif kind == 2:                          # truncate
        del b[rng.randrange(len(b) + 1):]
    elif kind == 3:                          # append
        b += bytes(rng.randrange(256) for _ in range(rng.randint(1, 64)))
    else:                                    # splice a piece of another stream
        o = rng.choice(bases)
        i, j = sorted(rng.randrange(len(o) + 1) for _ in range(2))
        k = rng.randrange(len(b) + 1)
        b[k:k] = o[i:j]
    return bytes(b)


bad = 0
n = int(sys.argv[3]) if len(sys.argv) > 3 else 3000
for it in range(n):
    s = rng.choice(bases)
    for _ in range(rng.randint(1, 3)):
        s = mutate(s)
    if rng.random() < 0.7:
        s = s[:len(s) - len(s) % 8]          # keep the length a multiple of 8 ...
    if rng.random() < 0.6:
        s = rehash(s)                        # ... and get past the checksum to the structure checks
    arr = (ctypes.c_uint8 * max(len(s), 1)).from_buffer_copy(s + b"\0")
    h = ctypes.c_void_p()
    rc = lib.adam_state_load(ctypes.byref(h), ctypes.cast(arr, ctypes.c_void_p), len(s), None)
    if rc == 0:
        lib.adam_state_destroy(h)
    elif rc not in (-1, -4, -5):
        print(f"iteration {it}: unexpected status {rc}: {B.adam_last_error()}")
        bad += 1
print(f"fuzzed {n} streams, {bad} unexpected results")
sys.exit(1 if bad else 0)
