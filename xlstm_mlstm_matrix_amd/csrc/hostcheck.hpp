// hostcheck.hpp -- host-side argument checks shared by the C ABI's entry
// points: address ranges of buffers, their overlap, alignment, size overflow.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

namespace mlstm {

struct Range {
    uintptr_t lo, hi;  // [lo, hi); empty when lo == hi
};
inline Range rng(const void *p, size_t bytes) {
    uintptr_t a = (uintptr_t)p;
    return Range{a, p ? a + bytes : a};
}
inline bool overlaps(Range a, Range b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}
inline bool same(Range a, Range b) { return a.lo == b.lo && a.hi == b.hi && a.lo < a.hi; }

// every pointer (NULL allowed) 16-byte aligned
inline bool all_aligned(std::initializer_list<const void *> ps) {
    for (const void *p : ps)
        if ((uintptr_t)p & 15) return false;
    return true;
}

inline bool mul_ok(size_t a, size_t b, size_t *out) {
    if (a != 0 && b > SIZE_MAX / a) return false;
    *out = a * b;
    return true;
}

}  // namespace mlstm
