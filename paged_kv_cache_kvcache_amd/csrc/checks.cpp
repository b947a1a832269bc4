// The device-data check switch and the error word query (the kernels' side of the checks lives in
// each kernel translation unit, next to the values it validates).
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "pkv_internal.h"

namespace pkv {

// -1: not decided yet (the environment decides on first use)
static std::atomic<int> g_device_checks{-1};

int device_checks() {
    int v = g_device_checks.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* e = std::getenv("PKV_CHECK");
        v = e != nullptr && std::strcmp(e, "1") == 0;
        int expected = -1;
        g_device_checks.compare_exchange_strong(expected, v);
        v = g_device_checks.load(std::memory_order_relaxed);
    }
    return v;
}

}  // namespace pkv

extern "C" int pkv_set_device_checks(int32_t enable) {
    pkv::g_device_checks.store(enable != 0 ? 1 : 0, std::memory_order_relaxed);
    return PKV_OK;
}

extern "C" int pkv_device_error(int32_t* code, int32_t* where, int32_t* value, void* stream) {
    PKV_REQUIRE(code != nullptr, PKV_ERR_INVALID, "code is NULL");
    int32_t first[3] = {0, 0, 0};
    int (*const readers[])(void*, int32_t*) = {pkv::read_error_kv_store, pkv::read_error_copy_blocks,
                                                pkv::read_error_decode, pkv::read_error_prefill};
    for (auto read : readers) {
        int32_t w[3] = {0, 0, 0};
        const int rc = read(stream, w);
        if (rc != PKV_OK) return rc;
        if (first[0] == 0 && w[0] != 0) std::memcpy(first, w, sizeof first);
    }
    *code = first[0];
    if (where) *where = first[1];
    if (value) *value = first[2];
    return PKV_OK;
}
