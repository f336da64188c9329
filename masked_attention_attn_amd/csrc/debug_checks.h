// Host-side consistency checks of the launch arithmetic: grid sizes, LDS bytes, and the
// extents every launcher derives from the validated sizes (32-bit buffer ranges and
// offsets, workspace layout).  Compiled in only with -DATTN_DEBUG (the debug build the
// host-sanitizer test makes); a failed check prints the condition and aborts.  The release
// build compiles them out: the API layer has already refused every size they guard.
#pragma once

#ifdef ATTN_DEBUG
#include <cstdio>
#include <cstdlib>
#define ATTN_CHECK(cond, what)                                                                     \
    do {                                                                                           \
        if (!(cond)) {                                                                             \
            std::fprintf(stderr, "ATTN_DEBUG check failed at %s:%d: %s (%s)\n", __FILE__, __LINE__, \
                         #cond, what);                                                             \
            std::abort();                                                                          \
        }                                                                                          \
    } while (0)
#else
#define ATTN_CHECK(cond, what) \
    do {                       \
    } while (0)
#endif

namespace mattn {
constexpr long long kLdsBytesPerCu = 160 * 1024;   // gfx950
constexpr long long kMaxGrid = (1ll << 31) - 1;
}  // namespace mattn
