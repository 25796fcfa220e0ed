"""Per-call routing digests: FNV-1a (64-bit) over every token's sorted expert
ids, so two runs of one layer compare with one string comparison (vllm.cpp PR
#2556, section "Why a value tap could never have said this").  The ids are
sorted because the assertion between two runs is set equality.  Reading: the
hash runs token-major over little-endian int32 ids."""
import numpy as np

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3


def fnv1a64(data: bytes) -> int:
    h = FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def route_digest(ids: np.ndarray) -> str:
    s = np.sort(np.asarray(ids, dtype=np.int32), axis=1).astype("<i4")
    return "%016x" % fnv1a64(s.tobytes())


def categorize(ids_a: np.ndarray, ids_b: np.ndarray):
    """Per token: identical (same ranked ids), order-only (same set, other
    ranking), or set-differs ("Batch changed the model's mind", section "16% of
    routing decisions")."""
    same = np.all(ids_a == ids_b, axis=1)
    same_set = np.all(np.sort(ids_a, axis=1) == np.sort(ids_b, axis=1), axis=1)
    return {
        "identical": int(same.sum()),
        "order_only": int((same_set & ~same).sum()),
        "set_differs": int((~same_set).sum()),
    }
