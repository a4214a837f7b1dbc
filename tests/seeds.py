"""Seeds for parametrised test cases that do not change between processes
(Python's hash() of a str is salted per process)."""
import zlib


def stable_seed(*parts) -> int:
    return zlib.crc32(repr(parts).encode())
