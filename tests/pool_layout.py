"""Byte positions of the pool's FP8 index-key page, written out from the layout that
include/dsa.h states (the tests' own copy; the generator and the library each have theirs)."""
import numpy as np


def fp8_key_positions(slot: int) -> np.ndarray:
    """Offsets, from the start of a block's FP8 key page, of bytes 0..127 of slot `slot`'s key:
    byte b at 2048 (slot / 16) + 1024 (b / 64) + 256 ((b / 16) % 4) + 16 (slot % 16) + b % 16."""
    b = np.arange(128)
    return (2048 * (slot // 16) + 1024 * (b // 64) + 256 * ((b // 16) % 4) + 16 * (slot % 16)
            + b % 16)
