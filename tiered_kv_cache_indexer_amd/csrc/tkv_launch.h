// Host-side launchers of the tiered KV-cache kernels.
#pragma once
#include "tkv_dev.h"

struct SelArgs;
struct StoreArgs;
struct AttnArgs;

hipError_t launch_select_scan(const DevCtx& c, const SelArgs& a, hipStream_t st);
hipError_t launch_select_rows(const DevCtx& c, const SelArgs& a, hipStream_t st);
hipError_t launch_prefill_scores(const DevCtx& c, const SelArgs& a, hipStream_t st);
hipError_t launch_ensure(const DevCtx& c, const int32_t* needed, int W, const uint8_t* no_fetch,
                         int32_t* out_slots, int32_t* miss, int32_t* miss_count, hipStream_t st);
hipError_t launch_fetch(const DevCtx& c, const int32_t* miss, const int32_t* miss_count, int width,
                        hipStream_t st);
hipError_t launch_fetch_slice(const DevCtx& c, const int32_t* miss, const int32_t* miss_count, int width, int s0,
                              int s1, int32_t* keep, hipStream_t st);
hipError_t launch_fetch_rest(const DevCtx& c, const int32_t* keep, int width, int sa, int sb, hipStream_t st);
hipError_t launch_write_ensure(const DevCtx& c, int n_runs, const int32_t* run_req,
                               const int32_t* run_start, const int32_t* run_len, int spr,
                               const int32_t* bt, int max_pages, const int32_t* old_len,
                               hipStream_t st);
hipError_t launch_store(const DevCtx& c, const StoreArgs& a, int max_run_len, hipStream_t st);
hipError_t launch_mirror_copy(const DevCtx& c, int layer, int blocks, hipStream_t st);
hipError_t launch_attn(const DevCtx& c, AttnArgs a, hipStream_t st);
bool attn_mfma_supported(const DevCtx& c);
hipError_t launch_attn_mfma(const DevCtx& c, AttnArgs a, hipStream_t st);
// the matrix-core split kernel serves `rows` decode rows (a folded fetch is possible)
bool attn_mfma_split_applies(const DevCtx& c, int rows);
hipError_t launch_reset(const DevCtx& c, int full, hipStream_t st);
hipError_t launch_fill_bytes(void* p, int64_t n, uint8_t v, hipStream_t st);
hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t st);
hipError_t launch_e4m3_decode(const uint8_t* in, float* out, int64_t n, hipStream_t st);
size_t select_dyn_lds(const DevCtx& c);
void prefix_copy_rows(uint8_t* dst, size_t dst_stride, const uint8_t* src, size_t src_stride, size_t row_bytes,
                      const int32_t* pages, int n, bool to_mirror, int max_threads);
hipError_t launch_slab_gather(const DevCtx& c, const int32_t* pages, int n, uint16_t* vals, double* sums,
                              hipStream_t st);
hipError_t launch_slab_scatter(const DevCtx& c, const int32_t* pages, int n, const uint16_t* vals,
                               const double* sums, hipStream_t st);
hipError_t launch_unbind(const DevCtx& c, const int32_t* pages, int n, hipStream_t st);
