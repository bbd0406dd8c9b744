#include <algorithm>
#include <vector>
// C ABI of the tiered KV-cache library: validation, buffer layout, launches.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/tkv.h"
#include "tkv_dev.h"
#include "tkv_launch.h"


// Staging memory of tkv_prefix_restore_noalloc: a file-scope device array,
// one copy per GPU, held until the process ends.  Host code never passes
// `scratch` itself to a kernel or a copy (on the host the name is only a
// stand-in): it uses the device address hipGetSymbolAddress returns, taken
// once per device when the first ctx attaches there.
#define TKV_SCRATCH_BYTES (2u << 20)
static __device__ __align__(256) uint8_t scratch[TKV_SCRATCH_BYTES];
#define TKV_MAX_DEVICES 64
static void* g_scratch_ptr[TKV_MAX_DEVICES];
static std::mutex g_scratch_mu[TKV_MAX_DEVICES];   // one restore at a time per device in this process

struct tkv_ctx {
  tkv_config cfg;
  int device = -1;      // the device current at tkv_attach_device
  size_t row_bytes, layer_bytes, code_bytes;
  size_t mirror_bytes;
  uint8_t* mirror_host = nullptr;
  uint8_t* mirror_dev = nullptr;
  bool attached = false;
  DevCtx dev{};
  int C = 0;            // compaction width (set_select_width)
  hipEvent_t ev_pre = nullptr, ev_copy = nullptr;   // preload ordering (created on first use)
  // Split decode copies (tkv_decode_layer_split).  Call k of a chain copies
  // its layer's and the next layer's slices on the caller's stream (ev_slice
  // after them), then the rest of the rows on the copy stream (ev_rest[k & 1]
  // after it), from miss-list copy k & 1.  rest_last indexes the latest
  // ev_rest; rest_cap is the capture sequence it was recorded in (0: none);
  // last_split is cleared by every other call.
  hipEvent_t ev_slice = nullptr, ev_rest[2] = {nullptr, nullptr};
  bool rest_pending = false, last_split = false;
  unsigned long long rest_cap = 0;
  // Split store (tkv_store_kv_mirror_split): the staged mirror blocks are
  // copied on the caller's copy stream; ev_mirror follows the latest copy,
  // recorded in capture sequence mirror_cap (0: none).  An eager split
  // store defers that copy (mdefer): the next attention call enqueues it
  // beside itself, any call that needs the mirror before that enqueues it
  // first; dev.stage_layer stays set until the next store, so that ensures
  // meanwhile patch staged blocks into the rows they fetch.
  hipEvent_t ev_mstage = nullptr, ev_mirror = nullptr;
  bool mirror_pending = false;
  unsigned long long mirror_cap = 0;
  bool mdefer = false;
  int mdefer_layer = 0, mdefer_blocks = 0;
  hipStream_t mdefer_s = nullptr, mdefer_cs = nullptr;
  int rest_last = 0, chain_len = 0, prev_layer = -1, prev_width = 0;
};

static thread_local std::string g_err;

static int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
static int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

static int hip_fail(hipError_t e, const char* what) {
  return fail(TKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIPCHECK(expr, what)                 \
  do {                                       \
    hipError_t e_ = (expr);                  \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t row, layer, code;
  size_t pool, slab, mirror;
  // state offsets
  size_t st_hdr, st_p2s, st_mark, st_s2p, st_stamp, st_order, st_acc, st_total;
  // workspace offsets
  size_t ws_scores, ws_sel_slots, ws_qg, ws_row_done, ws_glob, ws_slot_of_j, ws_miss_j, ws_victims, ws_wneeded,
      ws_wnofetch, ws_wmiss, ws_wmiss_count, ws_part, ws_attn_done, ws_iota, ws_sel_bm, ws_pout, ws_pmiss, ws_pmiss_count, ws_bg_miss, ws_stage, ws_stage_page, ws_rest_ctr, ws_miss_flag, ws_attn_state, ws_total;
  size_t stage_blocks;
};

static int validate(const tkv_config* c) {
  if (!c) return fail(TKV_E_INVALID_ARG, "config is NULL");
  if (c->kv_format == TKV_KV_NVFP4_BLOCK)
    return fail(TKV_E_UNSUPPORTED_FORMAT,
                "kv_format=nvfp4: per-block scales are not held by the host mirror rows; "
                "use kv_format=fp8_e4m3_per_token or bf16");
  if (c->kv_format != TKV_KV_BF16 && c->kv_format != TKV_KV_FP8_E4M3_PER_TOKEN)
    return fail(TKV_E_UNSUPPORTED_FORMAT, "kv_format=%d is not a known KV format", c->kv_format);
  if (c->num_layers < 1) return fail(TKV_E_INVALID_ARG, "num_layers=%d must be >= 1", c->num_layers);
  if (c->head_dim != 128) return fail(TKV_E_INVALID_ARG, "head_dim=%d: only 128 is supported", c->head_dim);
  if (c->num_kv_heads < 1 || c->num_q_heads != 8 * c->num_kv_heads)
    return fail(TKV_E_INVALID_ARG, "num_q_heads=%d, num_kv_heads=%d: the GQA group must be 8",
                c->num_q_heads, c->num_kv_heads);
  const int e8 = c->num_kv_heads * c->head_dim / 8;
  if (e8 != 16 && e8 != 32 && e8 != 64 && e8 != 128)
    return fail(TKV_E_INVALID_ARG, "num_kv_heads=%d: 1, 2, 4 or 8 KV heads are supported", c->num_kv_heads);
  if (c->page_size != 16 && c->page_size != 64)
    return fail(TKV_E_INVALID_ARG, "page_size=%d: 16 or 64 tokens are supported", c->page_size);
  if (c->num_logical_pages < 1 || c->num_logical_pages > 0x7FFFFFFF)
    return fail(TKV_E_INVALID_ARG, "num_logical_pages=%lld out of range", (long long)c->num_logical_pages);
  if (c->num_slots < 1 || c->num_slots > (1 << 19))
    return fail(TKV_E_INVALID_ARG, "num_slots=%d out of [1, 524288] (the ensure keeps one LDS bit per slot)",
                c->num_slots);
  if (c->max_batch < 1 || c->max_rows < c->max_batch)
    return fail(TKV_E_INVALID_ARG, "max_batch=%d, max_rows=%d: need 1 <= max_batch <= max_rows",
                c->max_batch, c->max_rows);
  if (c->max_topk < 1 || c->max_topk > 1024)
    return fail(TKV_E_INVALID_ARG, "max_topk=%d out of [1, 1024]", c->max_topk);
  if (c->max_pages_per_req < 1 || c->max_pages_per_req > 16384)
    return fail(TKV_E_INVALID_ARG, "max_pages_per_req=%d out of [1, 16384]", c->max_pages_per_req);
  if (c->max_width < 1 || c->max_width > 65535)
    return fail(TKV_E_INVALID_ARG, "max_width=%d out of [1, 65535]", c->max_width);
  return TKV_OK;
}

static Layout make_layout(const tkv_config* c) {
  Layout L{};
  const size_t H = c->num_kv_heads, PS = c->page_size, D = c->head_dim, N = c->num_logical_pages,
               S = c->num_slots, NL = c->num_layers;
  const bool fp8 = c->kv_format == TKV_KV_FP8_E4M3_PER_TOKEN;
  L.code = H * PS * D * (fp8 ? 1 : 2);
  L.layer = 2 * L.code + (fp8 ? 8 * PS : 0);
  L.row = NL * L.layer;
  L.pool = S * L.row;
  L.mirror = N * L.row;
  L.slab = NL * N * H * D * 2;
  size_t o = 0;
  L.st_hdr = o; o = align256(o + sizeof(StateHdr));
  L.st_p2s = o; o = align256(o + N * 4);
  L.st_mark = o; o = align256(o + N * 4);
  L.st_s2p = o; o = align256(o + S * 4);
  L.st_stamp = o; o = align256(o + S * 8);
  L.st_order = o; o = align256(o + 2 * S * 4);
  L.st_acc = o; o = align256(o + NL * N * H * D * 8);
  L.st_total = o;
  const size_t W = c->max_width, R = c->max_rows, P = c->max_pages_per_req;
  o = 0;
  L.ws_scores = o; o = align256(o + R * ((P + 63) / 64) * 64 * 8);
  L.ws_sel_slots = o; o = align256(o + R * (size_t)c->max_topk * 4);
  L.ws_qg = o; o = align256(o + R * H * D * 2);
  L.ws_row_done = o; o = align256(o + R * 4);
  L.ws_glob = o; o = align256(o + 16);
  L.ws_slot_of_j = o; o = align256(o + W * 4);
  L.ws_miss_j = o; o = align256(o + W * 4);
  L.ws_victims = o; o = align256(o + W * 4);
  L.ws_wneeded = o; o = align256(o + W * 4);
  L.ws_wnofetch = o; o = align256(o + W);
  L.ws_wmiss = o; o = align256(o + W * 8);
  L.ws_wmiss_count = o; o = align256(o + 4);
  L.ws_part = o; o = align256(o + (size_t)c->max_batch * c->num_q_heads * c->max_topk * (D + 4) * 4);
  L.ws_attn_done = o; o = align256(o + (size_t)c->max_batch * H * 4);
  L.ws_iota = o; o = align256(o + (R + 1) * 4);
  L.ws_sel_bm = o; o = align256(o + sel_bm_words(R, c->max_batch, P) * 4);
  L.ws_pout = o; o = align256(o + W * 4);
  L.ws_pmiss = o; o = align256(o + W * 8);
  L.ws_pmiss_count = o; o = align256(o + 4);
  L.ws_bg_miss = o; o = align256(o + 2 * (1 + 2 * W) * 4);
  // split store staging: one run of max_rows tokens (its pages plus the
  // boundary block the store grid adds)
  L.stage_blocks = (R + PS - 1) / PS + 1;
  L.ws_stage = o; o = align256(o + L.stage_blocks * L.layer);
  L.ws_stage_page = o; o = align256(o + L.stage_blocks * 4);
  L.ws_rest_ctr = o; o = align256(o + 8);
  L.ws_miss_flag = o; o = align256(o + W);
  // records of the page-range prefill attention: only configs with more rows than requests
  L.ws_attn_state = o;
  if (c->max_rows > c->max_batch) o = align256(o + R * (size_t)H * ATTN_STATE_FLOATS * 4);
  L.ws_total = o;
  return L;
}

extern "C" {

const char* tkv_last_error(void) { return g_err.c_str(); }

int tkv_required_bytes(const tkv_config* cfg, tkv_sizes* out) {
  int rc = validate(cfg);
  if (rc) return rc;
  if (!out) return fail(TKV_E_INVALID_ARG, "out is NULL");
  Layout L = make_layout(cfg);
  out->pool_bytes = L.pool;
  out->slab_bytes = L.slab;
  out->state_bytes = L.st_total;
  out->workspace_bytes = L.ws_total;
  out->mirror_bytes = L.mirror;
  out->row_bytes = L.row;
  out->layer_bytes = L.layer;
  return TKV_OK;
}

int tkv_create(const tkv_config* cfg, tkv_ctx** out) {
  int rc = validate(cfg);
  if (rc) return rc;
  if (!out) return fail(TKV_E_INVALID_ARG, "out is NULL");
  Layout L = make_layout(cfg);
  tkv_ctx* c = new tkv_ctx();
  c->cfg = *cfg;
  c->row_bytes = L.row;
  c->layer_bytes = L.layer;
  c->code_bytes = L.code;
  c->mirror_bytes = L.mirror;
  void* h = nullptr;
  hipError_t e = hipHostMalloc(&h, L.mirror, hipHostMallocMapped | hipHostMallocPortable);
  if (e != hipSuccess || !h) {
    delete c;
    return fail(TKV_E_OOM, "pinned host mirror of %zu bytes (num_logical_pages=%lld): %s", L.mirror,
                (long long)cfg->num_logical_pages, hipGetErrorString(e));
  }
  memset(h, 0, L.mirror);
  void* d = nullptr;
  e = hipHostGetDevicePointer(&d, h, 0);
  if (e != hipSuccess) {
    hipHostFree(h);
    delete c;
    return hip_fail(e, "hipHostGetDevicePointer(mirror)");
  }
  c->mirror_host = (uint8_t*)h;
  c->mirror_dev = (uint8_t*)d;
  *out = c;
  return TKV_OK;
}

void tkv_destroy(tkv_ctx* c) {
  if (!c) return;
  if (c->ev_pre) hipEventDestroy(c->ev_pre);
  if (c->ev_copy) hipEventDestroy(c->ev_copy);
  for (hipEvent_t e : c->ev_rest)
    if (e) hipEventSynchronize(e);
  // a deferred mirror copy is dropped with the mirror
  if (c->ev_mirror && c->mirror_pending) hipEventSynchronize(c->ev_mirror);
  for (hipEvent_t e : {c->ev_slice, c->ev_rest[0], c->ev_rest[1], c->ev_mstage, c->ev_mirror})
    if (e) hipEventDestroy(e);
  if (c->mirror_host) hipHostFree(c->mirror_host);
  delete c;
}

const void* tkv_mirror_host_ptr(const tkv_ctx* c) { return c ? c->mirror_host : nullptr; }

static bool aligned256(const void* p) { return ((uintptr_t)p & 255) == 0; }

int tkv_attach_device(tkv_ctx* c, const tkv_device_buffers* b, void* stream) {
  if (!c || !b) return fail(TKV_E_INVALID_ARG, "ctx or buffers is NULL");
  if (!b->pool || !b->slab || !b->state || !b->workspace)
    return fail(TKV_E_INVALID_ARG, "a device buffer is NULL (pool, slab, state, workspace)");
  if (!aligned256(b->pool) || !aligned256(b->slab) || !aligned256(b->state) || !aligned256(b->workspace))
    return fail(TKV_E_INVALID_ARG, "device buffers must be 256-byte aligned");
  Layout L = make_layout(&c->cfg);
  const tkv_config& f = c->cfg;
  DevCtx& d = c->dev;
  d = DevCtx{};
  d.L = f.num_layers; d.Hq = f.num_q_heads; d.Hkv = f.num_kv_heads; d.D = f.head_dim;
  d.PS = f.page_size; d.fp8 = f.kv_format == TKV_KV_FP8_E4M3_PER_TOKEN;
  d.N = f.num_logical_pages; d.S = f.num_slots;
  d.row_bytes = (int64_t)L.row; d.layer_bytes = (int64_t)L.layer; d.code_bytes = (int64_t)L.code;
  d.pool = (uint8_t*)b->pool;
  d.mirror = c->mirror_dev;
  d.slab = (uint16_t*)b->slab;
  uint8_t* st = (uint8_t*)b->state;
  d.hdr = (StateHdr*)(st + L.st_hdr);
  d.page_to_slot = (int32_t*)(st + L.st_p2s);
  d.page_mark = (int32_t*)(st + L.st_mark);
  d.slot_to_page = (int32_t*)(st + L.st_s2p);
  d.stamp = (int64_t*)(st + L.st_stamp);
  d.order = (int32_t*)(st + L.st_order);
  d.slab_acc = (double*)(st + L.st_acc);
  uint8_t* ws = (uint8_t*)b->workspace;
  d.scores = (float*)(ws + L.ws_scores);
  d.sel_slots = (int32_t*)(ws + L.ws_sel_slots);
  d.qg = (uint16_t*)(ws + L.ws_qg);
  d.row_done = (int32_t*)(ws + L.ws_row_done);
  d.glob_done = (int32_t*)(ws + L.ws_glob);
  d.slot_of_j = (int32_t*)(ws + L.ws_slot_of_j);
  d.miss_j = (int32_t*)(ws + L.ws_miss_j);
  d.victims = (int32_t*)(ws + L.ws_victims);
  d.wneeded = (int32_t*)(ws + L.ws_wneeded);
  d.wnofetch = (uint8_t*)(ws + L.ws_wnofetch);
  d.wmiss = (int32_t*)(ws + L.ws_wmiss);
  d.wmiss_count = (int32_t*)(ws + L.ws_wmiss_count);
  d.attn_part = (float*)(ws + L.ws_part);
  d.attn_done = (int32_t*)(ws + L.ws_attn_done);
  d.iota = (int32_t*)(ws + L.ws_iota);
  d.sel_bm = (uint32_t*)(ws + L.ws_sel_bm);
  d.pout = (int32_t*)(ws + L.ws_pout);
  d.pmiss = (int32_t*)(ws + L.ws_pmiss);
  d.pmiss_count = (int32_t*)(ws + L.ws_pmiss_count);
  d.bg_miss = (int32_t*)(ws + L.ws_bg_miss);
  d.stage = ws + L.ws_stage;
  d.stage_page = (int32_t*)(ws + L.ws_stage_page);
  d.stage_blocks = (int)L.stage_blocks;
  d.rest_ctr = (int32_t*)(ws + L.ws_rest_ctr);
  d.miss_flag = ws + L.ws_miss_flag;
  d.stage_layer = -1;
  d.stage_n = 0;
  d.attn_state = f.max_rows > f.max_batch ? (float*)(ws + L.ws_attn_state) : nullptr;
  d.attn_range_pages = ATTN_RANGE_PAGES_DEFAULT;
  d.max_rows = f.max_rows; d.max_pages = f.max_pages_per_req; d.max_topk = f.max_topk;
  d.max_batch = f.max_batch; d.max_width = f.max_width;
  int dev = 0;
  HIPCHECK(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= TKV_MAX_DEVICES) return fail(TKV_E_INVALID_ARG, "device %d >= %d", dev, TKV_MAX_DEVICES);
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu[dev]);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      HIPCHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
      g_scratch_ptr[dev] = p;
    }
  }
  c->device = dev;
  hipStream_t s = (hipStream_t)stream;
  HIPCHECK(launch_reset(d, 1, s), "initialise device state");
  HIPCHECK(hipStreamSynchronize(s), "hipStreamSynchronize");
  c->attached = true;
  return TKV_OK;
}

int tkv_set_select_width(tkv_ctx* c, int32_t max_bs, int32_t block_topk, int32_t max_sel_pages) {
  if (!c) return fail(TKV_E_INVALID_ARG, "ctx is NULL");
  if (max_bs < 1 || max_bs > c->cfg.max_batch)
    return fail(TKV_E_INVALID_ARG, "max_bs=%d out of [1, max_batch=%d]", max_bs, c->cfg.max_batch);
  if (block_topk < 1 || block_topk > c->cfg.max_topk)
    return fail(TKV_E_INVALID_ARG, "block_topk=%d out of [1, max_topk=%d]", block_topk, c->cfg.max_topk);
  const int C = max_sel_pages > 0 ? max_sel_pages : 2 * block_topk + 8;
  if ((int64_t)max_bs * C > c->cfg.num_slots)
    return fail(TKV_E_CAPACITY, "max_bs*max_sel_pages=%d*%d=%lld > num_slots=%d: the batch selection "
                "must fit the pool", max_bs, C, (long long)max_bs * C, c->cfg.num_slots);
  if ((int64_t)max_bs * C > c->cfg.max_width)
    return fail(TKV_E_CAPACITY, "max_bs*max_sel_pages=%lld > max_width=%d", (long long)max_bs * C,
                c->cfg.max_width);
  c->C = C;
  return TKV_OK;
}

int32_t tkv_select_width(const tkv_ctx* c) { return c ? c->C : 0; }

static int need_attached(tkv_ctx* c) {
  if (!c) return fail(TKV_E_INVALID_ARG, "ctx is NULL");
  if (!c->attached) return fail(TKV_E_STATE, "device buffers not attached (tkv_attach_device)");
  return TKV_OK;
}

// Capture sequence `s` records into (0 when it is not capturing).
static unsigned long long capture_id(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  unsigned long long id = 0;
  if (hipStreamGetCaptureInfo(s, &st, &id) != hipSuccess || st != hipStreamCaptureStatusActive) return 0;
  return id;
}

// Orders `s` after the last rest-of-rows copy of a split decode call.  A copy
// recorded in another capture sequence (or outside the one `s` records into)
// is not waited for: a graph holds only its own work, and the caller orders
// graphs against eager work.
//
// It also orders `s` after the latest staged mirror copy of a split store:
// every call that waits here reads or writes the mirror or the pool (the
// selection and the ensure do neither and run beside that copy).
// Enqueues a deferred mirror copy on the copy stream of its store, ordered
// after `s` when `s` is the store's stream and records eagerly (then the copy
// starts where the caller is now, e.g. beside the attention it is about to
// launch), else after the store's stream as it stands.
static int launch_deferred_mirror(tkv_ctx* c, hipStream_t s) {
  if (!c->mdefer) return TKV_OK;
  hipStream_t rs = (s == c->mdefer_s && capture_id(s) == 0) ? s : c->mdefer_s;
  if (capture_id(rs) != 0)
    return fail(TKV_E_STATE, "a split store's mirror copy is pending on a stream now being captured "
                             "(call tkv_mirror_flush before the capture)");
  c->mdefer = false;
  HIPCHECK(hipEventRecord(c->ev_mstage, rs), "hipEventRecord");
  HIPCHECK(hipStreamWaitEvent(c->mdefer_cs, c->ev_mstage, 0), "hipStreamWaitEvent");
  HIPCHECK(launch_mirror_copy(c->dev, c->mdefer_layer, c->mdefer_blocks, c->mdefer_cs), "mirror copy launch");
  HIPCHECK(hipEventRecord(c->ev_mirror, c->mdefer_cs), "hipEventRecord");
  c->mirror_pending = true;
  c->mirror_cap = 0;
  return TKV_OK;
}

static int wait_mirror(tkv_ctx* c, hipStream_t s) {
  int rc = launch_deferred_mirror(c, s);
  if (rc) return rc;
  if (c->mirror_pending && capture_id(s) == c->mirror_cap) {
    HIPCHECK(hipStreamWaitEvent(s, c->ev_mirror, 0), "hipStreamWaitEvent(mirror copy)");
    // from here on `s` sees the staged blocks in the mirror (which a later
    // prefix restore may overwrite): nothing left to patch
    c->dev.stage_layer = -1;
    c->dev.stage_n = 0;
  }
  return TKV_OK;
}

// Orders `s` after the last rest-of-rows copy only: for fetches (the ensure
// that produced their miss list patched any staged block into the rows they
// read) and attention that reads the pool only.
static int wait_rest_copy(tkv_ctx* c, hipStream_t s) {
  c->last_split = false;
  if (!c->rest_pending || capture_id(s) != c->rest_cap) return TKV_OK;
  HIPCHECK(hipStreamWaitEvent(s, c->ev_rest[c->rest_last], 0), "hipStreamWaitEvent(rest copy)");
  return TKV_OK;
}

static int wait_rest(tkv_ctx* c, hipStream_t s) {
  int rc = wait_mirror(c, s);
  if (rc) return rc;
  return wait_rest_copy(c, s);
}

// The copies of a split decode call, issued after its selection and ensure
// (which ran beside earlier copies: they touch no pool bytes and no kept
// miss list).  W is the call's ensure width.  On `s`: the slices of this
// layer and of the next one, for every miss; on `cs`: the rest of the rows.
//
// A call chains on the previous one when that was the ctx's last call, for
// the layer before, and num_slots >= W_prev + 2*W: then no slot the previous
// call filled is rebound by this call's ensure (at least num_slots - W_prev
// - W slots outside both calls are older and the misses take at most W of
// them).  Its slice copy then waits only for the rest copy of the call two
// back (whose slots this call may rebind, and whose kept list it reuses).
// Its attention reads this layer's slice of pages missed here (copied just
// before), by the previous call (copied there as that call's next slice) or
// earlier (rest copies two or more back: done).  Anything else waits for
// every earlier copy.
static int split_copies(tkv_ctx* c, int layer, const int32_t* miss, const int32_t* miss_count, int W,
                        hipStream_t s, hipStream_t cs) {
  const unsigned long long cap = capture_id(s);
  const int L = c->cfg.num_layers;
  const bool same = c->rest_pending && cap == c->rest_cap;
  const bool chained = same && c->last_split && layer == (c->prev_layer + 1) % L &&
                       (int64_t)c->cfg.num_slots >= (int64_t)c->prev_width + 2 * (int64_t)W;
  if (!chained) {
    if (same) HIPCHECK(hipStreamWaitEvent(s, c->ev_rest[c->rest_last], 0), "hipStreamWaitEvent(rest copy)");
    c->chain_len = 0;
  } else if (c->chain_len >= 2) {
    HIPCHECK(hipStreamWaitEvent(s, c->ev_rest[c->rest_last ^ 1], 0), "hipStreamWaitEvent(rest copy, two back)");
  }
  const int k = c->chain_len & 1;
  int32_t* keep = c->dev.bg_miss + (size_t)k * (1 + 2 * (size_t)c->cfg.max_width);
  // (the copies read the mirror rows of this call's misses, which its
  // ensure completed from any staged blocks: no wait for a mirror copy)
  const int nxt = (layer + 1) % L;
  HIPCHECK(launch_fetch_slice(c->dev, miss, miss_count, W, layer, nxt, keep, s), "decode slice fetch launch");
  HIPCHECK(hipEventRecord(c->ev_slice, s), "hipEventRecord");
  HIPCHECK(hipStreamWaitEvent(cs, c->ev_slice, 0), "hipStreamWaitEvent");
  HIPCHECK(launch_fetch_rest(c->dev, keep, W, layer, nxt, cs), "rest-of-rows fetch launch");
  HIPCHECK(hipEventRecord(c->ev_rest[k], cs), "hipEventRecord");
  c->rest_last = k;
  c->rest_pending = true;
  c->rest_cap = cap;
  c->chain_len += 1;
  c->prev_layer = layer;
  c->prev_width = W;
  c->last_split = true;
  return TKV_OK;
}

#define WAIT_REST(c, s)                                \
  do {                                                 \
    int rc_ = wait_rest((c), (hipStream_t)(s));        \
    if (rc_) return rc_;                               \
  } while (0)

#define WAIT_REST_COPY(c, s)                           \
  do {                                                 \
    int rc_ = wait_rest_copy((c), (hipStream_t)(s));   \
    if (rc_) return rc_;                               \
  } while (0)

int tkv_reset_residency(tkv_ctx* c, void* stream) {
  int rc = need_attached(c);
  if (rc) return rc;
  WAIT_REST(c, stream);
  HIPCHECK(launch_reset(c->dev, 0, (hipStream_t)stream), "reset residency");
  return TKV_OK;
}

static int check_rows(tkv_ctx* c, int layer, int rows, int B, int max_pages, int topk) {
  const tkv_config& f = c->cfg;
  if (layer < 0 || layer >= f.num_layers) return fail(TKV_E_INVALID_ARG, "layer=%d out of [0, %d)", layer, f.num_layers);
  if (rows < 1 || rows > f.max_rows) return fail(TKV_E_INVALID_ARG, "rows=%d out of [1, max_rows=%d]", rows, f.max_rows);
  if (B < 1 || B > f.max_batch) return fail(TKV_E_INVALID_ARG, "B=%d out of [1, max_batch=%d]", B, f.max_batch);
  if (max_pages < 1 || max_pages > f.max_pages_per_req)
    return fail(TKV_E_INVALID_ARG, "max_pages=%d out of [1, max_pages_per_req=%d]", max_pages, f.max_pages_per_req);
  if (topk < 1 || topk > f.max_topk) return fail(TKV_E_INVALID_ARG, "topk=%d out of [1, max_topk=%d]", topk, f.max_topk);
  return TKV_OK;
}

// bf16 rows (queries, new keys and values) are read in 16-byte vectors
static int check_vec16(const void* p, const char* name) {
  if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0)
    return fail(TKV_E_INVALID_ARG, "%s=%p is not 16-byte aligned", name, p);
  return TKV_OK;
}

static SelArgs make_sel(tkv_ctx* c, int layer, const uint16_t* q, int rows, const int32_t* row_start,
                        const int32_t* row_pos, const int32_t* bt, int max_pages, const int32_t* n_pages,
                        int B, const float* bias, int topk, int32_t* sel, int32_t* needed) {
  SelArgs a{};
  a.layer = layer; a.q = q; a.rows = rows; a.row_start = row_start; a.row_pos = row_pos;
  a.bt = bt; a.max_pages = max_pages; a.n_pages = n_pages; a.B = B; a.bias = bias; a.topk = topk;
  a.sel_local = sel; a.needed = needed; a.C = c->C;
  a.n_chunks = (max_pages + SEL_CHUNK - 1) / SEL_CHUNK;
  return a;
}

int tkv_select_pages(tkv_ctx* c, int32_t layer, const uint16_t* q, int32_t rows, const int32_t* row_start,
                     const int32_t* row_pos, const int32_t* block_table, int32_t max_pages,
                     const int32_t* n_pages, int32_t B, const float* page_bias, int32_t topk,
                     int32_t* sel_local, int32_t* needed, void* stream) {
  int rc = need_attached(c);
  if (rc) return rc;
  if ((rc = check_rows(c, layer, rows, B, max_pages, topk))) return rc;
  if (!c->C) return fail(TKV_E_STATE, "select width not set (tkv_set_select_width)");
  if (!q || !row_start || !block_table || !n_pages || !sel_local || !needed)
    return fail(TKV_E_INVALID_ARG, "a required pointer is NULL (q, row_start, block_table, n_pages, sel_local, needed)");
  if ((rc = check_vec16(q, "q"))) return rc;
  SelArgs a = make_sel(c, layer, q, rows, row_start, row_pos, block_table, max_pages, n_pages, B,
                       page_bias, topk, sel_local, needed);
  a.do_ensure = 0;
  c->last_split = false;
  if (row_pos && B == 1 && rows >= 64) {
    // a chunk of query rows of one request: indexer scores as a matrix product
    HIPCHECK(launch_prefill_scores(c->dev, a, (hipStream_t)stream), "select_pages (prefill) launch");
  } else {
    HIPCHECK(launch_select_scan(c->dev, a, (hipStream_t)stream), "select_pages launch");
  }
  return TKV_OK;
}

int tkv_lru_ensure(tkv_ctx* c, const int32_t* needed, int32_t width, const uint8_t* no_fetch,
                   int32_t* out_slots, int32_t* miss, int32_t* miss_count, void* stream) {
  int rc = need_attached(c);
  if (rc) return rc;
  if (width < 1 || width > c->cfg.max_width)
    return fail(TKV_E_INVALID_ARG, "width=%d out of [1, max_width=%d]", width, c->cfg.max_width);
  if (!needed || !miss || !miss_count)
    return fail(TKV_E_INVALID_ARG, "needed, miss and miss_count must not be NULL");
  c->last_split = false;   // an ensure between split calls voids their no-rebind argument
  HIPCHECK(launch_ensure(c->dev, needed, width, no_fetch, out_slots, miss, miss_count, (hipStream_t)stream),
           "lru_ensure launch");
  return TKV_OK;
}

int tkv_fetch_pages(tkv_ctx* c, const int32_t* miss, const int32_t* miss_count, int32_t width, void* stream) {
  int rc = need_attached(c);
  if (rc) return rc;
  if (width < 1 || !miss || !miss_count) return fail(TKV_E_INVALID_ARG, "miss, miss_count or width invalid");
  WAIT_REST_COPY(c, stream);
  HIPCHECK(launch_fetch(c->dev, miss, miss_count, width, (hipStream_t)stream), "fetch_pages launch");
  return TKV_OK;
}

int tkv_fetch_pages_layer(tkv_ctx* c, const int32_t* miss, const int32_t* miss_count, int32_t width, int32_t layer,
                          void* stream) {
  int rc = need_attached(c);
  if (rc) return rc;
  if (width < 1 || width > c->cfg.max_width || !miss || !miss_count)
    return fail(TKV_E_INVALID_ARG, "miss, miss_count or width (must be in [1, max_width=%d]) invalid",
                c->cfg.max_width);
  if (layer < 0 || layer >= c->cfg.num_layers) return fail(TKV_E_INVALID_ARG, "layer=%d out of range", layer);
  WAIT_REST_COPY(c, stream);
  HIPCHECK(launch_fetch_slice(c->dev, miss, miss_count, width, layer, layer, c->dev.bg_miss, (hipStream_t)stream),
           "fetch_pages_layer launch");
  return TKV_OK;
}

int tkv_fetch_pages_rest(tkv_ctx* c, int32_t width, int32_t layer, void* stream) {
  int rc = need_attached(c);
  if (rc) return rc;
  if (width < 1 || width > c->cfg.max_width)
    return fail(TKV_E_INVALID_ARG, "width=%d out of [1, max_width=%d]", width, c->cfg.max_width);
  if (layer < 0 || layer >= c->cfg.num_layers) return fail(TKV_E_INVALID_ARG, "layer=%d out of range", layer);
  WAIT_REST_COPY(c, stream);
  HIPCHECK(launch_fetch_rest(c->dev, c->dev.bg_miss, width, layer, layer, (hipStream_t)stream),
           "fetch_pages_rest launch");
  return TKV_OK;
}

static int attn_call(tkv_ctx* c, int32_t layer, const uint16_t* q, int32_t rows, const int32_t* row_start,
                     const int32_t* row_pos, const int32_t* ctx_len, int32_t B, const int32_t* sel_local,
                     const int32_t* block_table, int32_t max_pages, int32_t topk, uint16_t* out, void* stream,
                     int host_tail) {
  int rc = need_attached(c);
  if (rc) return rc;
  if ((rc = check_rows(c, layer, rows, B, max_pages, topk))) return rc;
  if (!q || !row_start || !ctx_len || !sel_local || !block_table || !out)
    return fail(TKV_E_INVALID_ARG, "a required pointer is NULL (q, row_start, ctx_len, sel_local, block_table, out)");
  if ((rc = check_vec16(q, "q")) || (rc = check_vec16(out, "out"))) return rc;
  if (rows > c->cfg.max_batch && topk > 64)
    return fail(TKV_E_INVALID_ARG, "topk=%d > 64 with rows=%d > max_batch: such rows are not split", topk, rows);
  AttnArgs a{};
  a.layer = layer; a.q = q; a.rows = rows; a.row_start = row_start; a.row_pos = row_pos;
  a.ctx_len = ctx_len; a.sel = sel_local; a.bt = block_table; a.max_pages = max_pages; a.topk = topk;
  a.B = B; a.out = out; a.host_tail = host_tail;
  if (host_tail) {
    WAIT_REST(c, stream);                        // reads mirror rows
  } else {
    // reads the pool only: a deferred mirror copy starts beside it
    if ((rc = launch_deferred_mirror(c, (hipStream_t)stream))) return rc;
    WAIT_REST_COPY(c, stream);
  }
  HIPCHECK(launch_attn(c->dev, a, (hipStream_t)stream), "sparse_paged_attn launch");
  return TKV_OK;
}

int tkv_sparse_paged_attn(tkv_ctx* c, int32_t layer, const uint16_t* q, int32_t rows,
                          const int32_t* row_start, const int32_t* row_pos, const int32_t* ctx_len,
                          int32_t B, const int32_t* sel_local, const int32_t* block_table,
                          int32_t max_pages, int32_t topk, uint16_t* out, void* stream) {
  return attn_call(c, layer, q, rows, row_start, row_pos, ctx_len, B, sel_local, block_table, max_pages, topk,
                   out, stream, 0);
}

int tkv_sparse_paged_attn_host_tail(tkv_ctx* c, int32_t layer, const uint16_t* q, int32_t rows,
                                    const int32_t* row_start, const int32_t* row_pos, const int32_t* ctx_len,
                                    int32_t B, const int32_t* sel_local, const int32_t* block_table,
                                    int32_t max_pages, int32_t topk, uint16_t* out, void* stream) {
  return attn_call(c, layer, q, rows, row_start, row_pos, ctx_len, B, sel_local, block_table, max_pages, topk,
                   out, stream, 1);
}

static int decode_layer_impl(tkv_ctx* c, int32_t layer, const uint16_t* q, int32_t B,
                             const int32_t* block_table, int32_t max_pages, const int32_t* n_pages,
                             const int32_t* ctx_len, const float* page_bias, int32_t topk, int32_t* sel_local,
                             int32_t* needed, int32_t* out_slots, int32_t* miss, int32_t* miss_count,
                             uint16_t* out, const int32_t* pred, int32_t pred_width, void* stream,
                             void* copy_stream, bool split) {
  int rc = need_attached(c);
  if (rc) return rc;
  if ((rc = check_rows(c, layer, B, B, max_pages, topk))) return rc;
  if (!c->C) return fail(TKV_E_STATE, "select width not set (tkv_set_select_width)");
  if (!q || !block_table || !n_pages || !ctx_len || !sel_local || !needed || !out_slots || !miss || !miss_count || !out)
    return fail(TKV_E_INVALID_ARG, "a required pointer is NULL");
  if ((rc = check_vec16(q, "q")) || (rc = check_vec16(out, "out"))) return rc;
  if ((int64_t)B * c->C > c->cfg.max_width || (int64_t)B * c->C > c->cfg.num_slots)
    return fail(TKV_E_CAPACITY, "B*max_sel_pages=%lld exceeds num_slots or max_width", (long long)B * c->C);
  hipStream_t s = (hipStream_t)stream;
  hipStream_t cs = (hipStream_t)copy_stream;
  const bool overlap = pred && cs && cs != s;
  split = split && c->cfg.num_layers > 1;   // one layer: the slice is the row
  if (split && !c->ev_slice) {
    for (hipEvent_t* e : {&c->ev_slice, &c->ev_rest[0], &c->ev_rest[1]})
      HIPCHECK(hipEventCreateWithFlags(e, hipEventDisableTiming), "hipEventCreate");
  }
  if (pred) {
    WAIT_REST(c, s);
    if (pred_width < 1 || pred_width > c->cfg.max_width || pred_width > c->cfg.num_slots)
      return fail(TKV_E_INVALID_ARG, "pred_width=%d out of [1, min(max_width=%d, num_slots=%d)]", pred_width,
                  c->cfg.max_width, c->cfg.num_slots);
    if (overlap && !c->ev_pre) {
      HIPCHECK(hipEventCreateWithFlags(&c->ev_pre, hipEventDisableTiming), "hipEventCreate");
      HIPCHECK(hipEventCreateWithFlags(&c->ev_copy, hipEventDisableTiming), "hipEventCreate");
    }
    HIPCHECK(launch_ensure(c->dev, pred, pred_width, nullptr, c->dev.pout, c->dev.pmiss, c->dev.pmiss_count, s),
             "preload ensure launch");
    if (overlap) {
      HIPCHECK(hipEventRecord(c->ev_pre, s), "hipEventRecord");
      HIPCHECK(hipStreamWaitEvent(cs, c->ev_pre, 0), "hipStreamWaitEvent");
      HIPCHECK(launch_fetch(c->dev, c->dev.pmiss, c->dev.pmiss_count, pred_width, cs), "preload fetch launch");
      HIPCHECK(hipEventRecord(c->ev_copy, cs), "hipEventRecord");
    } else {
      HIPCHECK(launch_fetch(c->dev, c->dev.pmiss, c->dev.pmiss_count, pred_width, s), "preload fetch launch");
    }
  }
  SelArgs a = make_sel(c, layer, q, B, c->dev.iota, nullptr, block_table, max_pages, n_pages, B,
                       page_bias, topk, sel_local, needed);
  a.do_ensure = 1;
  a.one_row_each = 1;
  a.out_slots = out_slots;
  a.miss = miss;
  a.miss_count = miss_count;
  // one row per request: with topk <= C a row's selection is its request's
  // needed list in order, so the ensure's out_slots are the slots the
  // attention reads (row stride C); otherwise a translated copy
  const bool direct = topk <= c->C;
  a.sel_slots = direct ? nullptr : c->dev.sel_slots;
  // one stream, matrix-core split attention: the fetch is folded into the
  // attention launch (its pages of this layer read from their mirror rows)
  const bool fold = !split && direct && attn_mfma_split_applies(c->dev, B);
  a.miss_flag = fold ? c->dev.miss_flag : nullptr;
  HIPCHECK(launch_select_scan(c->dev, a, s), "decode select+ensure launch");
  // the layer's ensure may have rebound a slot the preload copy still writes:
  // its own fetch (and the attention) wait for that copy
  if (overlap) HIPCHECK(hipStreamWaitEvent(s, c->ev_copy, 0), "hipStreamWaitEvent");
  if (split) {
    if ((rc = split_copies(c, layer, miss, miss_count, B * c->C, s, cs))) return rc;
  } else {
    // the selection and ensure ran beside a split call's copies (they touch
    // no pool bytes and no kept miss list); the copy waits for them
    WAIT_REST_COPY(c, s);
    if (!fold) HIPCHECK(launch_fetch(c->dev, miss, miss_count, B * c->C, s), "decode fetch launch");
  }
  if ((rc = launch_deferred_mirror(c, s))) return rc;   // beside the attention
  AttnArgs t{};
  t.layer = layer; t.q = q; t.rows = B; t.row_start = c->dev.iota; t.row_pos = nullptr;
  t.ctx_len = ctx_len; t.sel = sel_local; t.bt = block_table; t.max_pages = max_pages; t.topk = topk;
  t.B = B; t.out = out;
  t.one_row_each = 1;
  t.slots = direct ? out_slots : c->dev.sel_slots;
  t.slots_stride = direct ? c->C : 0;
  if (fold) {
    t.fmiss = miss;
    t.fmiss_count = miss_count;
    t.fwidth = B * c->C;
    t.slot_miss = c->dev.miss_flag;
    t.slot_page = needed;   // a row's selection is its request's needed list, in order
  }
  HIPCHECK(launch_attn(c->dev, t, s), fold ? "decode attention+fetch launch" : "decode attention launch");
  return TKV_OK;
}

int tkv_decode_layer(tkv_ctx* c, int32_t layer, const uint16_t* q, int32_t B, const int32_t* block_table,
                     int32_t max_pages, const int32_t* n_pages, const int32_t* ctx_len,
                     const float* page_bias, int32_t topk, int32_t* sel_local, int32_t* needed,
                     int32_t* out_slots, int32_t* miss, int32_t* miss_count, uint16_t* out, void* stream) {
  return decode_layer_impl(c, layer, q, B, block_table, max_pages, n_pages, ctx_len, page_bias, topk, sel_local,
                           needed, out_slots, miss, miss_count, out, nullptr, 0, stream, nullptr, false);
}

int tkv_decode_layer_split(tkv_ctx* c, int32_t layer, const uint16_t* q, int32_t B, const int32_t* block_table,
                           int32_t max_pages, const int32_t* n_pages, const int32_t* ctx_len,
                           const float* page_bias, int32_t topk, int32_t* sel_local, int32_t* needed,
                           int32_t* out_slots, int32_t* miss, int32_t* miss_count, uint16_t* out, void* stream,
                           void* copy_stream) {
  return decode_layer_impl(c, layer, q, B, block_table, max_pages, n_pages, ctx_len, page_bias, topk, sel_local,
                           needed, out_slots, miss, miss_count, out, nullptr, 0, stream, copy_stream, true);
}

int tkv_decode_layer_prefetch(tkv_ctx* c, int32_t layer, const uint16_t* q, int32_t B,
                              const int32_t* block_table, int32_t max_pages, const int32_t* n_pages,
                              const int32_t* ctx_len, const float* page_bias, int32_t topk, int32_t* sel_local,
                              int32_t* needed, int32_t* out_slots, int32_t* miss, int32_t* miss_count,
                              uint16_t* out, const int32_t* pred, int32_t pred_width, void* stream,
                              void* copy_stream) {
  if (!pred) return fail(TKV_E_INVALID_ARG, "pred is NULL");
  return decode_layer_impl(c, layer, q, B, block_table, max_pages, n_pages, ctx_len, page_bias, topk, sel_local,
                           needed, out_slots, miss, miss_count, out, pred, pred_width, stream, copy_stream,
                           false);
}

int tkv_ensure_write_pages(tkv_ctx* c, int32_t n_runs, const int32_t* run_req, const int32_t* run_start,
                           const int32_t* run_len, int32_t max_run_len, const int32_t* block_table,
                           int32_t max_pages, const int32_t* old_len, void* stream) {
  int rc = need_attached(c);
  if (rc) return rc;
  if (n_runs < 1 || max_run_len < 1) return fail(TKV_E_INVALID_ARG, "n_runs=%d, max_run_len=%d must be >= 1", n_runs, max_run_len);
  if (!run_req || !run_start || !run_len || !block_table || !old_len)
    return fail(TKV_E_INVALID_ARG, "a required pointer is NULL");
  if (max_pages < 1 || max_pages > c->cfg.max_pages_per_req) return fail(TKV_E_INVALID_ARG, "max_pages out of range");
  const int spr = (max_run_len + c->cfg.page_size - 1) / c->cfg.page_size + 1;
  if ((int64_t)n_runs * spr > c->cfg.max_width)
    return fail(TKV_E_CAPACITY, "n_runs*(max_run_len/page_size+1)=%lld samples > max_width=%d",
                (long long)n_runs * spr, c->cfg.max_width);
  WAIT_REST(c, stream);
  HIPCHECK(launch_write_ensure(c->dev, n_runs, run_req, run_start, run_len, spr, block_table, max_pages,
                               old_len, (hipStream_t)stream), "ensure_write_pages launch");
  return TKV_OK;
}

static int store_impl(tkv_ctx* c, int32_t layer, const uint16_t* k, const uint16_t* v, int32_t n_runs,
                      const int32_t* run_req, const int32_t* run_start, const int32_t* run_len,
                      const int32_t* run_tok_off, int32_t max_run_len, const int32_t* block_table,
                      int32_t max_pages, void* stream, void* copy_stream, bool split) {
  int rc = need_attached(c);
  if (rc) return rc;
  if (layer < 0 || layer >= c->cfg.num_layers) return fail(TKV_E_INVALID_ARG, "layer=%d out of range", layer);
  if (n_runs < 1 || max_run_len < 1) return fail(TKV_E_INVALID_ARG, "n_runs=%d, max_run_len=%d must be >= 1", n_runs, max_run_len);
  if (!k || !v || !run_req || !run_start || !run_len || !run_tok_off || !block_table)
    return fail(TKV_E_INVALID_ARG, "a required pointer is NULL");
  if ((rc = check_vec16(k, "k")) || (rc = check_vec16(v, "v"))) return rc;
  if (max_pages < 1 || max_pages > c->cfg.max_pages_per_req) return fail(TKV_E_INVALID_ARG, "max_pages out of range");
  StoreArgs a{};
  a.layer = layer; a.k = k; a.v = v; a.n_runs = n_runs; a.run_req = run_req; a.run_start = run_start;
  a.run_len = run_len; a.run_tok_off = run_tok_off; a.bt = block_table; a.max_pages = max_pages;
  hipStream_t s = (hipStream_t)stream, cs = (hipStream_t)copy_stream;
  WAIT_REST(c, s);   // also the previous split store's copy, which read the staging buffer
  c->dev.stage_layer = -1;   // ... so its staged blocks are in the mirror from here on
  c->dev.stage_n = 0;
  if (!split || !cs || cs == s) {
    HIPCHECK(launch_store(c->dev, a, max_run_len, s), "store_kv_mirror launch");
    return TKV_OK;
  }
  if (!c->ev_mirror) {
    HIPCHECK(hipEventCreateWithFlags(&c->ev_mstage, hipEventDisableTiming), "hipEventCreate");
    HIPCHECK(hipEventCreateWithFlags(&c->ev_mirror, hipEventDisableTiming), "hipEventCreate");
  }
  const int ppr = (max_run_len + c->cfg.page_size - 1) / c->cfg.page_size + 1;
  const int64_t blocks = (int64_t)n_runs * ppr;
  a.stage = c->dev.stage;
  a.stage_page = c->dev.stage_page;
  a.stage_blocks = c->dev.stage_blocks;
  HIPCHECK(launch_store(c->dev, a, max_run_len, s), "store_kv_mirror_split launch");
  const int nb = (int)std::min<int64_t>(blocks, c->dev.stage_blocks);
  c->dev.stage_layer = layer;
  c->dev.stage_n = nb;
  const unsigned long long cap = capture_id(s);
  if (cap == 0) {
    // eager: the copy waits for the next attention call (or a call that needs the mirror)
    c->mdefer = true;
    c->mdefer_layer = layer;
    c->mdefer_blocks = nb;
    c->mdefer_s = s;
    c->mdefer_cs = cs;
    return TKV_OK;
  }
  HIPCHECK(hipEventRecord(c->ev_mstage, s), "hipEventRecord");
  HIPCHECK(hipStreamWaitEvent(cs, c->ev_mstage, 0), "hipStreamWaitEvent");
  HIPCHECK(launch_mirror_copy(c->dev, layer, nb, cs), "mirror copy launch");
  HIPCHECK(hipEventRecord(c->ev_mirror, cs), "hipEventRecord");
  c->mirror_pending = true;
  c->mirror_cap = cap;
  return TKV_OK;
}

int tkv_store_kv_mirror(tkv_ctx* c, int32_t layer, const uint16_t* k, const uint16_t* v, int32_t n_runs,
                        const int32_t* run_req, const int32_t* run_start, const int32_t* run_len,
                        const int32_t* run_tok_off, int32_t max_run_len, const int32_t* block_table,
                        int32_t max_pages, void* stream) {
  return store_impl(c, layer, k, v, n_runs, run_req, run_start, run_len, run_tok_off, max_run_len, block_table,
                    max_pages, stream, nullptr, false);
}

int tkv_mirror_flush(tkv_ctx* c, void* stream) {
  int rc = need_attached(c);
  if (rc) return rc;
  return wait_mirror(c, (hipStream_t)stream);
}

int tkv_store_kv_mirror_split(tkv_ctx* c, int32_t layer, const uint16_t* k, const uint16_t* v, int32_t n_runs,
                              const int32_t* run_req, const int32_t* run_start, const int32_t* run_len,
                              const int32_t* run_tok_off, int32_t max_run_len, const int32_t* block_table,
                              int32_t max_pages, void* stream, void* copy_stream) {
  return store_impl(c, layer, k, v, n_runs, run_req, run_start, run_len, run_tok_off, max_run_len, block_table,
                    max_pages, stream, copy_stream, true);
}

int tkv_read_counters(tkv_ctx* c, tkv_counters* out, void* stream) {
  int rc = need_attached(c);
  if (rc) return rc;
  if (!out) return fail(TKV_E_INVALID_ARG, "out is NULL");
  StateHdr h;
  hipStream_t s = (hipStream_t)stream;
  WAIT_REST(c, s);
  HIPCHECK(hipMemcpyAsync(&h, c->dev.hdr, sizeof h, hipMemcpyDeviceToHost, s), "read counters");
  HIPCHECK(hipStreamSynchronize(s), "hipStreamSynchronize");
  out->ensure_calls = h.counters[CNT_ENSURE];
  out->hits = h.counters[CNT_HITS];
  out->misses = h.counters[CNT_MISSES];
  out->fresh_allocs = h.counters[CNT_FRESH];
  out->evictions = h.counters[CNT_EVICT];
  out->drops = h.counters[CNT_DROPS];
  out->bytes_fetched = h.counters[CNT_BYTES_FETCHED];
  out->bytes_mirrored = h.counters[CNT_BYTES_MIRRORED];
  out->clock = h.clock;
  out->error_word = h.error_word;
  out->reserved = 0;
  return TKV_OK;
}

int tkv_debug_read_state(tkv_ctx* c, int32_t* page_to_slot, int32_t* slot_to_page, int64_t* stamp,
                         int64_t* clock, void* stream) {
  int rc = need_attached(c);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  WAIT_REST(c, s);
  const DevCtx& d = c->dev;
  if (page_to_slot) HIPCHECK(hipMemcpyAsync(page_to_slot, d.page_to_slot, (size_t)d.N * 4, hipMemcpyDeviceToHost, s), "read page_to_slot");
  if (slot_to_page) HIPCHECK(hipMemcpyAsync(slot_to_page, d.slot_to_page, (size_t)d.S * 4, hipMemcpyDeviceToHost, s), "read slot_to_page");
  if (stamp) HIPCHECK(hipMemcpyAsync(stamp, d.stamp, (size_t)d.S * 8, hipMemcpyDeviceToHost, s), "read stamp");
  StateHdr h;
  HIPCHECK(hipMemcpyAsync(&h, d.hdr, sizeof h, hipMemcpyDeviceToHost, s), "read clock");
  HIPCHECK(hipStreamSynchronize(s), "hipStreamSynchronize");
  if (clock) *clock = h.clock;
  return TKV_OK;
}

int64_t tkv_prefix_record_bytes(const tkv_ctx* c) {
  if (!c) return 0;
  const int64_t E = (int64_t)c->cfg.num_kv_heads * c->cfg.head_dim;
  return (int64_t)c->row_bytes + (int64_t)c->cfg.num_layers * E * 10;
}

static int check_prefix_pages(tkv_ctx* c, const int32_t* pages, int32_t n, bool distinct) {
  int rc = need_attached(c);
  if (rc) return rc;
  if (!pages || n < 1) return fail(TKV_E_INVALID_ARG, "pages is NULL or n=%d < 1", n);
  for (int i = 0; i < n; ++i)
    if (pages[i] < 0 || (int64_t)pages[i] >= c->cfg.num_logical_pages)
      return fail(TKV_E_INVALID_ARG, "pages[%d]=%d out of [0, num_logical_pages=%lld)", i, pages[i],
                  (long long)c->cfg.num_logical_pages);
  if (distinct) {
    std::vector<int32_t> v(pages, pages + n);
    std::sort(v.begin(), v.end());
    if (std::adjacent_find(v.begin(), v.end()) != v.end())
      return fail(TKV_E_INVALID_ARG, "pages has duplicates");
  }
  return TKV_OK;
}

// Slab entries of `n` pages between records and the device, 128 pages at a time.
static int prefix_slab(tkv_ctx* c, const int32_t* pages, int32_t n, uint8_t* recs, bool save, hipStream_t s) {
  const size_t E = (size_t)c->cfg.num_kv_heads * c->cfg.head_dim, L = c->cfg.num_layers;
  const size_t rec = (size_t)tkv_prefix_record_bytes(c), vbytes = L * E * 2, sbytes = L * E * 8;
  const int SLICE = 128;
  const int m = std::min(n, SLICE);
  void* dev = nullptr;
  HIPCHECK(hipMalloc(&dev, m * (vbytes + sbytes) + (size_t)m * 4), "hipMalloc (prefix staging)");
  uint16_t* dv = (uint16_t*)dev;
  double* ds = (double*)((uint8_t*)dev + m * vbytes);
  int32_t* dp = (int32_t*)((uint8_t*)dev + m * (vbytes + sbytes));
  std::vector<uint8_t> host(m * (vbytes + sbytes));
  hipError_t e = hipSuccess;
  for (int i0 = 0; i0 < n && e == hipSuccess; i0 += SLICE) {
    const int k = std::min(SLICE, n - i0);
    e = hipMemcpyAsync(dp, pages + i0, (size_t)k * 4, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) break;
    if (save) {
      if ((e = launch_slab_gather(c->dev, dp, k, dv, ds, s)) != hipSuccess) break;
      if ((e = hipMemcpyAsync(host.data(), dv, k * vbytes, hipMemcpyDeviceToHost, s)) != hipSuccess) break;
      if ((e = hipMemcpyAsync(host.data() + m * vbytes, ds, k * sbytes, hipMemcpyDeviceToHost, s)) != hipSuccess)
        break;
      if ((e = hipStreamSynchronize(s)) != hipSuccess) break;
      for (int i = 0; i < k; ++i) {
        uint8_t* r = recs + (size_t)(i0 + i) * rec + c->row_bytes;
        memcpy(r, host.data() + (size_t)i * vbytes, vbytes);
        memcpy(r + vbytes, host.data() + m * vbytes + (size_t)i * sbytes, sbytes);
      }
    } else {
      for (int i = 0; i < k; ++i) {
        const uint8_t* r = recs + (size_t)(i0 + i) * rec + c->row_bytes;
        memcpy(host.data() + (size_t)i * vbytes, r, vbytes);
        memcpy(host.data() + m * vbytes + (size_t)i * sbytes, r + vbytes, sbytes);
      }
      if ((e = hipMemcpyAsync(dv, host.data(), k * vbytes, hipMemcpyHostToDevice, s)) != hipSuccess) break;
      if ((e = hipMemcpyAsync(ds, host.data() + m * vbytes, k * sbytes, hipMemcpyHostToDevice, s)) != hipSuccess)
        break;
      if ((e = launch_slab_scatter(c->dev, dp, k, dv, ds, s)) != hipSuccess) break;
      if ((e = launch_unbind(c->dev, dp, k, s)) != hipSuccess) break;
      if ((e = hipStreamSynchronize(s)) != hipSuccess) break;
    }
  }
  hipError_t e2 = hipStreamSynchronize(s);
  hipFree(dev);
  if (e == hipSuccess) e = e2;
  HIPCHECK(e, save ? "prefix save (slab)" : "prefix restore (slab, unbind)");
  return TKV_OK;
}

int tkv_prefix_save(tkv_ctx* c, const int32_t* pages, int32_t n, void* records, void* stream) {
  int rc = check_prefix_pages(c, pages, n, false);
  if (rc) return rc;
  if (!records) return fail(TKV_E_INVALID_ARG, "records is NULL");
  hipStream_t s = (hipStream_t)stream;
  WAIT_REST(c, s);
  HIPCHECK(hipStreamSynchronize(s), "hipStreamSynchronize");   // stores to the mirror have landed
  const size_t rec = (size_t)tkv_prefix_record_bytes(c);
  prefix_copy_rows((uint8_t*)records, rec, c->mirror_host, c->row_bytes, c->row_bytes, pages, n, false, 8);
  return prefix_slab(c, pages, n, (uint8_t*)records, true, s);
}

int tkv_prefix_restore(tkv_ctx* c, const int32_t* pages, int32_t n, const void* records, void* stream) {
  int rc = check_prefix_pages(c, pages, n, true);
  if (rc) return rc;
  if (!records) return fail(TKV_E_INVALID_ARG, "records is NULL");
  hipStream_t s = (hipStream_t)stream;
  WAIT_REST(c, s);
  HIPCHECK(hipStreamSynchronize(s), "hipStreamSynchronize");   // no copy still reads these rows
  const size_t rec = (size_t)tkv_prefix_record_bytes(c);
  prefix_copy_rows(c->mirror_host, c->row_bytes, (const uint8_t*)records, rec, c->row_bytes, pages, n, true, 8);
  return prefix_slab(c, pages, n, const_cast<uint8_t*>((const uint8_t*)records), false, s);
}

// Distinct ids without allocating anything: pairwise comparison.
static int check_prefix_pages_noalloc(tkv_ctx* c, const int32_t* pages, int32_t n) {
  int rc = check_prefix_pages(c, pages, n, false);
  if (rc) return rc;
  for (int i = 1; i < n; ++i)
    for (int j = 0; j < i; ++j)
      if (pages[i] == pages[j])
        return fail(TKV_E_INVALID_ARG, "pages has duplicates (pages[%d] == pages[%d] == %d)", j, i, pages[i]);
  return TKV_OK;
}

// Pages of slab entries one pass of the no-alloc restore stages: values
// [m][L][E] bf16, then (256-aligned) key sums [m][L][E] fp64, then (256-
// aligned) the page ids; 0 when one page does not fit.
static int noalloc_slice_pages(size_t vbytes, size_t sbytes) {
  for (int m = (int)(TKV_SCRATCH_BYTES / (vbytes + sbytes + 4)); m > 0; --m)
    if (align256(m * vbytes) + align256(m * sbytes) + (size_t)m * 4 <= TKV_SCRATCH_BYTES) return m;
  return 0;
}

int tkv_prefix_restore_noalloc(tkv_ctx* c, const int32_t* pages, int32_t n, const void* records, void* stream) {
  int rc = check_prefix_pages_noalloc(c, pages, n);
  if (rc) return rc;
  if (!records) return fail(TKV_E_INVALID_ARG, "records is NULL");
  const size_t E = (size_t)c->cfg.num_kv_heads * c->cfg.head_dim, L = c->cfg.num_layers;
  const size_t vbytes = L * E * 2, sbytes = L * E * 8;
  const int m = noalloc_slice_pages(vbytes, sbytes);
  if (m < 1)
    return fail(TKV_E_CAPACITY, "one page's slab entries (%zu bytes, num_layers=%d x num_kv_heads*head_dim=%zu) "
                "exceed the %u-byte staging array of the no-alloc restore", vbytes + sbytes + 4,
                c->cfg.num_layers, E, (unsigned)TKV_SCRATCH_BYTES);
  int cur = -1;
  HIPCHECK(hipGetDevice(&cur), "hipGetDevice");
  if (cur != c->device)
    return fail(TKV_E_STATE, "device %d is current; the ctx was attached on device %d", cur, c->device);
  uint8_t* base = (uint8_t*)g_scratch_ptr[c->device];
  if (!base) return fail(TKV_E_STATE, "no staging address for device %d", c->device);
  uint16_t* dv = (uint16_t*)base;
  double* ds = (double*)(base + align256(m * vbytes));
  int32_t* dp = (int32_t*)(base + align256(m * vbytes) + align256(m * sbytes));
  hipStream_t s = (hipStream_t)stream;
  WAIT_REST(c, s);
  HIPCHECK(hipStreamSynchronize(s), "hipStreamSynchronize");   // no copy still reads these rows
  const size_t rec = (size_t)tkv_prefix_record_bytes(c);
  const uint8_t* recs = (const uint8_t*)records;
  prefix_copy_rows(c->mirror_host, c->row_bytes, recs, rec, c->row_bytes, pages, n, true, 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu[c->device]);
  for (int i0 = 0; i0 < n; i0 += m) {
    const int k = std::min(m, n - i0);
    const uint8_t* r0 = recs + (size_t)i0 * rec + c->row_bytes;
    HIPCHECK(hipMemcpyAsync(dp, pages + i0, (size_t)k * 4, hipMemcpyHostToDevice, s), "restore: page ids");
    HIPCHECK(hipMemcpy2DAsync(dv, vbytes, r0, rec, vbytes, k, hipMemcpyHostToDevice, s), "restore: slab values");
    HIPCHECK(hipMemcpy2DAsync(ds, sbytes, r0 + vbytes, rec, sbytes, k, hipMemcpyHostToDevice, s), "restore: key sums");
    HIPCHECK(launch_slab_scatter(c->dev, dp, k, dv, ds, s), "restore: slab scatter");
    HIPCHECK(launch_unbind(c->dev, dp, k, s), "restore: unbind");
    HIPCHECK(hipStreamSynchronize(s), "hipStreamSynchronize");   // the next pass reuses the staging
  }
  return TKV_OK;
}

int tkv_debug_set_attn_kernel(tkv_ctx* c, int32_t kernel) {
  if (!c) return fail(TKV_E_INVALID_ARG, "ctx is null");
  if (kernel < TKV_ATTN_AUTO || kernel > TKV_ATTN_MATRIX)
    return fail(TKV_E_INVALID_ARG, "attention kernel=%d: expected 0 (auto), 1 (vector) or 2 (matrix)", kernel);
  if (kernel == TKV_ATTN_MATRIX) {
    const tkv_config& f = c->cfg;
    if (!(f.kv_format == TKV_KV_FP8_E4M3_PER_TOKEN && f.page_size == 64 && f.head_dim == 128 &&
          f.num_q_heads == 8 * f.num_kv_heads))
      return fail(TKV_E_UNSUPPORTED_FORMAT,
                  "the matrix-core attention kernel needs kv_format=fp8, page_size=64, head_dim=128, "
                  "8 query heads per KV head");
  }
  c->dev.attn_impl = kernel == TKV_ATTN_VECTOR ? ATTN_VECTOR : kernel == TKV_ATTN_MATRIX ? ATTN_MATRIX : ATTN_AUTO;
  return TKV_OK;
}

int tkv_debug_set_attn_range(tkv_ctx* c, int32_t pages) {
  if (!c) return fail(TKV_E_INVALID_ARG, "ctx is null");
  if (pages < 0) return fail(TKV_E_INVALID_ARG, "pages=%d < 0", pages);
  c->dev.attn_range_pages = pages;
  return TKV_OK;
}

int tkv_debug_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (!in || !out || n < 0) return fail(TKV_E_INVALID_ARG, "bad arguments");
  HIPCHECK(launch_e4m3_encode(in, out, n, (hipStream_t)stream), "e4m3 encode launch");
  return TKV_OK;
}

int tkv_debug_e4m3_decode(const uint8_t* in, float* out, int64_t n, void* stream) {
  if (!in || !out || n < 0) return fail(TKV_E_INVALID_ARG, "bad arguments");
  HIPCHECK(launch_e4m3_decode(in, out, n, (hipStream_t)stream), "e4m3 decode launch");
  return TKV_OK;
}

}  // extern "C"
