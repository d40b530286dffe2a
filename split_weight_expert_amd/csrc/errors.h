// Host-side helpers shared by the library's translation units: the thread-local error state and
// argument checks.  No HIP header is needed, so the host-only parts of the library (the slice plan,
// record layout, pointer table and workspace sizing in host.cpp) also build with a plain C++ compiler,
// e.g. for the sanitizer test of that logic.
#pragma once

#include <stdint.h>
#include <stddef.h>
#include <string>

#include "../../include/dwdp.h"

namespace dwdp {

// ---------------------------------------------------------------- host: errors
void set_error(const std::string& msg);
void clear_error();

struct Fail {
    int code;
};

inline int fail(int code, const std::string& msg) {
    set_error(msg);
    return code;
}

#define DWDP_REQUIRE(cond, msg)                                                       \
    do {                                                                              \
        if (!(cond)) return ::dwdp::fail(DWDP_ERR_INVALID_ARG, std::string(__func__) + ": " + (msg)); \
    } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kFp8Group = 128;     // activation group width and weight block edge
constexpr int kNumXcd = 8;         // MI355X: 8 accelerator complex dies, 32 CUs each

}  // namespace dwdp
