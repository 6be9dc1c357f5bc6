// The C ABI's enum parameters as the int they carry.  A C caller may pass any
// int for an enum parameter (C allows any value of the enum's integer type),
// while C++ may only load an enum-typed object holding a value in the range
// of its enumerators.  Every entry point therefore reads its enum arguments'
// bytes as an int and validates that, never the enum-typed value itself.
#pragma once

#include <stdint.h>
#include <string.h>

#include "tg.h"

namespace tg {

// Largest size or leading dimension (in elements) the library takes; larger
// ones return TG_ERR_NOT_SUPPORTED.  With every extent at most 2^31 - 1, all
// byte offsets and tile counts the host code forms fit in 64 bits.
constexpr int64_t kMaxDim = 0x7FFFFFFF;

inline bool dims_fit(int64_t a, int64_t b, int64_t c, int64_t d = 0, int64_t e = 0, int64_t f = 0)
{
    return a <= kMaxDim && b <= kMaxDim && c <= kMaxDim && d <= kMaxDim && e <= kMaxDim && f <= kMaxDim;
}

template <class E>
inline int abi_int(const E& e)
{
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized on this ABI");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}

}  // namespace tg
