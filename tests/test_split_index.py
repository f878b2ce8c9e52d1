"""CPU check of the split prefill's index arithmetic (tests/hip/split_check.hip,
compiled for the host from the kernels' own header): run boundaries and
their inverse, the interleaved query-tile order and its inverse, and the
workspace slots of cut tiles, over seeded random schedules."""
import ctypes
import os

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libsplit_check.so")


def test_split_runs_order_and_slots_are_consistent():
    assert os.path.exists(LIB), "split check library not built"
    lib = ctypes.CDLL(LIB)
    lib.split_check.argtypes = [ctypes.c_char_p, ctypes.c_int]
    buf = ctypes.create_string_buffer(256)
    failures = lib.split_check(buf, 256)
    assert failures == 0, buf.value.decode()
