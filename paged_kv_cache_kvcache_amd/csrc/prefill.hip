// Varlen paged prefill attention for gfx950 (bf16 MFMA).  Placeholder until the kernel lands.
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

extern "C" int pkv_paged_attn_prefill(const pkv_cache_desc* desc, const void* q, int32_t Hq,
                                      const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t B,
                                      int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                      int32_t max_blocks, float softmax_scale, int32_t causal, void* out,
                                      void* stream) {
    int rc = pkv::check_desc(desc);
    if (rc != PKV_OK) return rc;
    return pkv::fail(PKV_ERR_UNSUPPORTED, "prefill is not implemented yet");
}
