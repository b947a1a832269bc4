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

// Device-data checks: 1 when kernels validate the indices they read from device memory (slots,
// block ids, lengths, launch order, run lists) and report the first bad one in their translation
// unit's error word instead of using it.  Off unless PKV_CHECK=1 is set in the environment when
// the library first asks, or pkv_set_device_checks(1) was called.
int device_checks();

// Error word codes (pkv_device_error).
enum DeviceError : int32_t {
    kErrSlot = 1,       // slot outside the pool (>= num_blocks * 256)
    kErrBlock = 2,      // block id outside 0..num_blocks-1
    kErrLength = 3,     // context / key length outside what the block table can hold
    kErrSequence = 4,   // launch-order entry outside 0..B-1
    kErrRun = 5,        // run list entry outside the batch or its block
    kErrCuSeqlens = 6,  // cu_seqlens_q not non-decreasing within 0..total_q
    kErrRows = 7,       // copy row count outside 0..256
    kErrShared = 8,     // a group member whose block table differs within the group's shared keys
};

// Each kernel translation unit keeps its own error word (code, where, value) in device memory;
// these read it and clear it on `stream` (a hipStream_t), then wait for the stream.  Return 0 or
// a PKV_ERR_HIP code.
int read_error_kv_store(void* stream, int32_t* out);
int read_error_copy_blocks(void* stream, int32_t* out);
int read_error_decode(void* stream, int32_t* out);
int read_error_prefill(void* stream, int32_t* out);

}  // namespace pkv

#define PKV_REQUIRE(cond, code, ...)                 \
    do {                                             \
        if (!(cond)) return ::pkv::fail(code, __VA_ARGS__); \
    } while (0)
