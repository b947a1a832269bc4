// Internal helpers shared by the libpkv translation units (not part of the ABI).
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "pkv.h"

namespace pkv {

constexpr int kBlock = PKV_BLOCK_SIZE;

// Records the failure text for pkv_last_error() on this thread and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline int dtype_bytes(int32_t dt) {
    switch (dt) {
        case PKV_F32: return 4;
        case PKV_BF16: return 2;
        case PKV_I8: return 1;
        default: return 0;
    }
}

// Host-side checks shared by the device entry points.
int check_desc(const pkv_cache_desc* d);

}  // namespace pkv

#define PKV_REQUIRE(cond, code, ...)                 \
    do {                                             \
        if (!(cond)) return ::pkv::fail(code, __VA_ARGS__); \
    } while (0)
