"""CPU check of the LDS XOR swizzles the kernels use (tests/hip/swizzle_check.hip,
compiled for the host): each layout is a bijection with a correct inverse,
and every access group the kernels issue (16 rows of one 16-byte chunk
column; 4 rows x 4 chunks for transposed reads) covers the 16 distinct
16-byte slots of a 256-byte line."""
import ctypes
import os

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libswizzle_check.so")


def test_swizzles_are_bijective_and_conflict_free():
    assert os.path.exists(LIB), "swizzle check library not built"
    lib = ctypes.CDLL(LIB)
    lib.swizzle_check.argtypes = [ctypes.c_char_p, ctypes.c_int]
    buf = ctypes.create_string_buffer(256)
    failures = lib.swizzle_check(buf, 256)
    assert failures == 0, buf.value.decode()
