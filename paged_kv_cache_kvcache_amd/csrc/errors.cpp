// Thread-local error text behind pkv_last_error(), and checks shared by the entry points.
#include "pkv_internal.h"

namespace pkv {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

void clear_error() { g_last_error.clear(); }

int check_desc(const pkv_cache_desc* d) {
    PKV_REQUIRE(d != nullptr, PKV_ERR_INVALID, "cache descriptor is NULL");
    PKV_REQUIRE(d->block_size == kBlock, PKV_ERR_UNSUPPORTED, "block_size %d: only 256 is supported",
                d->block_size);
    PKV_REQUIRE(d->num_blocks > 0, PKV_ERR_INVALID, "num_blocks %d must be positive", d->num_blocks);
    PKV_REQUIRE(d->num_kv_heads > 0, PKV_ERR_INVALID, "num_kv_heads %d must be positive",
                d->num_kv_heads);
    PKV_REQUIRE(d->head_dim == 64 || d->head_dim == 128, PKV_ERR_UNSUPPORTED,
                "head_dim %d: only 64 and 128 are supported", d->head_dim);
    PKV_REQUIRE(dtype_bytes(d->kv_dtype) != 0, PKV_ERR_UNSUPPORTED, "unknown kv_dtype %d", d->kv_dtype);
    return PKV_OK;
}

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }

extern "C" const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }
