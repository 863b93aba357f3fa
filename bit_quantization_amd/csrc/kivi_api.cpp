// C ABI entry points: argument validation, per-layer views, launches.
// Nothing is enqueued unless every check passes; no C++ exception crosses the ABI.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include <atomic>
#include <mutex>

#include "../../include/kivi.h"
#include "kivi_internal.h"

namespace kivi {

int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1) {
    (void)hipGetLastError();
    return 256;
  }
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace kivi

namespace {

thread_local char g_err[512] = "";

kivi_status fail(kivi_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kivi_status ok() {
  g_err[0] = '\0';
  return KIVI_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_one_of(int v, std::initializer_list<int> set) {
  for (int x : set)
    if (v == x) return true;
  return false;
}

kivi_status check_dims(const kivi_dims* d) {
  if (!d) return fail(KIVI_ERR_ARG, "dims is NULL");
  if (d->layers < 1 || d->batch < 1 || d->kv_heads < 1 || d->q_heads < 1)
    return fail(KIVI_ERR_ARG, "layers, batch, kv_heads and q_heads must be >= 1");
  if ((int64_t)d->batch * d->kv_heads > 65535)
    return fail(KIVI_ERR_UNSUPPORTED, "batch * kv_heads = %lld exceeds 65535",
                (long long)d->batch * d->kv_heads);
  if (d->q_heads % d->kv_heads != 0)
    return fail(KIVI_ERR_ARG, "q_heads (%d) is not a multiple of kv_heads (%d)", d->q_heads,
                d->kv_heads);
  if (!is_one_of(d->q_heads / d->kv_heads, {1, 2, 4, 8}))
    return fail(KIVI_ERR_UNSUPPORTED, "q_heads / kv_heads = %d; supported: 1, 2, 4, 8",
                d->q_heads / d->kv_heads);
  if (d->bits != 2 && d->bits != 4)
    return fail(KIVI_ERR_UNSUPPORTED, "bits = %d; supported: 2, 4", d->bits);
  if (d->head_dim != kivi::kHeadDim)
    return fail(KIVI_ERR_UNSUPPORTED, "head_dim = %d; supported: %d", d->head_dim,
                kivi::kHeadDim);
  if (!is_one_of(d->group_k, {16, 32, 64}))
    return fail(KIVI_ERR_UNSUPPORTED, "group_k = %d; supported: 16, 32, 64", d->group_k);
  if (d->group_v < 1 || d->head_dim % d->group_v != 0)
    return fail(KIVI_ERR_ARG, "group_v = %d does not divide head_dim = %d", d->group_v,
                d->head_dim);
  if (!is_one_of(d->group_v, {16, 32, 64, 128}))
    return fail(KIVI_ERR_UNSUPPORTED, "group_v = %d; supported: 16, 32, 64, 128", d->group_v);
  if (d->residual < 1 || d->residual % d->group_k != 0 || d->residual % kivi::kVRun != 0)
    return fail(KIVI_ERR_ARG, "residual = %d must be a positive multiple of group_k (%d) and 16",
                d->residual, d->group_k);
  if (d->sink < 0 || d->sink > 1024)
    return fail(KIVI_ERR_ARG, "sink = %d outside [0, 1024]", d->sink);
  if (d->aging != KIVI_AGING_WINDOW && d->aging != KIVI_AGING_GROUP)
    return fail(KIVI_ERR_ARG, "aging = %d; expected KIVI_AGING_WINDOW (0) or KIVI_AGING_GROUP (1)",
                d->aging);
  if (d->flags & ~(KIVI_FLAG_VALUE_TOKEN_WINDOW | KIVI_FLAG_DETERMINISTIC))
    return fail(KIVI_ERR_ARG, "flags = 0x%x: unknown bits", (unsigned)d->flags);
  if (d->max_tokens < 1 || d->max_tokens % d->group_k != 0 || d->max_tokens % kivi::kVRun != 0)
    return fail(KIVI_ERR_ARG, "max_tokens = %lld must be a positive multiple of group_k and 16",
                (long long)d->max_tokens);
  // The kernels address one pair's history with 32-bit buffer offsets; the codes are
  // its largest buffer (d*b/8 bytes per token against at most 16 of scales).
  if (d->max_tokens > kivi::kMaxPairBytes / (d->head_dim * d->bits / 8))
    return fail(KIVI_ERR_UNSUPPORTED,
                "max_tokens = %lld: a pair's %d-bit codes would exceed %lld bytes (at most %lld "
                "tokens)", (long long)d->max_tokens, d->bits, (long long)kivi::kMaxPairBytes,
                (long long)(kivi::kMaxPairBytes / (d->head_dim * d->bits / 8)));
  return KIVI_OK;
}

// pg == nullptr: contiguous history, one section of max_tokens per (b, h); else one
// section per KV head holding the page pool.
void buffer_sizes(const kivi_dims* d, const kivi_paging* pg, size_t out[KIVI_NUM_BUFFERS]) {
  const size_t unit = (size_t)d->layers * d->batch * d->kv_heads;
  const size_t sections = pg ? (size_t)d->layers * d->kv_heads : unit;
  const size_t T = pg ? (size_t)pg->pages * pg->page_tokens : (size_t)d->max_tokens;
  const size_t codes = sections * T * d->head_dim * d->bits / 8;
  const size_t kmeta = sections * (T / d->group_k) * d->head_dim * 2;
  const size_t vmeta = sections * T * (d->head_dim / d->group_v) * 2;
  const size_t resid = unit * (size_t)(d->sink + d->residual) * d->head_dim * 2;
  out[0] = codes;
  out[1] = kmeta;
  out[2] = kmeta;
  out[3] = codes;
  out[4] = vmeta;
  out[5] = vmeta;
  out[6] = resid;
  out[7] = resid;
  out[8] = unit * 2 * sizeof(float);
}

kivi_status check_cache(const kivi_cache* c) {
  if (!c) return fail(KIVI_ERR_ARG, "cache is NULL");
  const void* p[KIVI_NUM_BUFFERS] = {c->k_codes, c->k_scale, c->k_zero,
                                     c->v_codes, c->v_scale, c->v_zero,
                                     c->k_resid, c->v_resid, c->scale_max};
  static const char* names[KIVI_NUM_BUFFERS] = {"k_codes", "k_scale", "k_zero",
                                                "v_codes", "v_scale", "v_zero",
                                                "k_resid", "v_resid", "scale_max"};
  for (int i = 0; i < KIVI_NUM_BUFFERS; ++i) {
    if (!p[i]) return fail(KIVI_ERR_ARG, "cache.%s is NULL", names[i]);
    if (!aligned16(p[i])) return fail(KIVI_ERR_ALIGN, "cache.%s is not 16-byte aligned", names[i]);
  }
  return KIVI_OK;
}

// The dims of a layer, no buffers (planning).
kivi::LayerView shape_view(const kivi_dims* d) {
  kivi::LayerView L{};
  L.B = d->batch;
  L.H = d->kv_heads;
  L.d = d->head_dim;
  L.bits = d->bits;
  L.G = d->group_k;
  L.Gv = d->group_v;
  L.R = d->residual;
  L.S = d->sink;
  L.aging = d->aging;
  L.vwin = (d->flags & KIVI_FLAG_VALUE_TOKEN_WINDOW) ? 1 : 0;
  L.det = (d->flags & KIVI_FLAG_DETERMINISTIC) ? 1 : 0;
  L.Tmax = d->max_tokens;
  return L;
}

kivi::LayerView layer_view(const kivi_dims* d, const kivi_cache* c, int layer,
                           const kivi_paging* pg = nullptr) {
  size_t sz[KIVI_NUM_BUFFERS];
  buffer_sizes(d, pg, sz);
  kivi::LayerView L = shape_view(d);
  if (pg) {
    L.table = pg->block_table;
    L.page_log2 = __builtin_ctz((unsigned)pg->page_tokens);
    L.pages_per_seq = pg->pages_per_seq;
    L.pages = pg->pages;
  }
  const size_t Ld = (size_t)d->layers;
  L.k_codes = static_cast<uint8_t*>(c->k_codes) + layer * (sz[0] / Ld);
  L.k_scale = reinterpret_cast<__half*>(static_cast<uint8_t*>(c->k_scale) + layer * (sz[1] / Ld));
  L.k_zero = reinterpret_cast<__half*>(static_cast<uint8_t*>(c->k_zero) + layer * (sz[2] / Ld));
  L.v_codes = static_cast<uint8_t*>(c->v_codes) + layer * (sz[3] / Ld);
  L.v_scale = reinterpret_cast<__half*>(static_cast<uint8_t*>(c->v_scale) + layer * (sz[4] / Ld));
  L.v_zero = reinterpret_cast<__half*>(static_cast<uint8_t*>(c->v_zero) + layer * (sz[5] / Ld));
  L.k_resid = reinterpret_cast<__half*>(static_cast<uint8_t*>(c->k_resid) + layer * (sz[6] / Ld));
  L.v_resid = reinterpret_cast<__half*>(static_cast<uint8_t*>(c->v_resid) + layer * (sz[7] / Ld));
  L.scale_max = reinterpret_cast<float*>(static_cast<uint8_t*>(c->scale_max) + layer * (sz[8] / Ld));
  return L;
}

// A paged cache: pages of a power-of-two number of tokens (>= 64, so that a decode
// block never straddles two), enough pages per sequence for max_tokens, and a page
// pool whose per-head byte offsets fit the 32-bit buffer offsets of the kernels.
kivi_status check_page_geometry(const kivi_dims* d, const kivi_paging* pg) {
  const int32_t P = pg->page_tokens;
  if (P < 64 || P > (1 << 20) || (P & (P - 1)) != 0)
    return fail(KIVI_ERR_ARG, "page_tokens = %d must be a power of two in [64, 2^20]", P);
  if (pg->pages < 1 || pg->pages_per_seq < 1)
    return fail(KIVI_ERR_ARG, "pages and pages_per_seq must be >= 1");
  if ((int64_t)pg->pages_per_seq * P < d->max_tokens)
    return fail(KIVI_ERR_CAPACITY, "pages_per_seq * page_tokens = %lld < max_tokens = %lld",
                (long long)pg->pages_per_seq * P, (long long)d->max_tokens);
  if (pg->pages * P * (int64_t)(d->head_dim * d->bits / 8) >= ((int64_t)1 << 31))
    return fail(KIVI_ERR_UNSUPPORTED, "a KV head's page pool holds 2^31 bytes or more");
  return KIVI_OK;
}

kivi_status check_paging(const kivi_dims* d, const kivi_paging* pg) {
  if (!pg) return KIVI_OK;
  kivi_status st = check_page_geometry(d, pg);
  if (st != KIVI_OK) return st;
  if (!pg->block_table) return fail(KIVI_ERR_ARG, "block_table is NULL");
  if ((reinterpret_cast<uintptr_t>(pg->block_table) & 3u) != 0)
    return fail(KIVI_ERR_ALIGN, "block_table is not 4-byte aligned");
  return KIVI_OK;
}

// The per-token Value window is built for uniform batches in contiguous caches.
kivi_status check_vwin(const kivi_dims* d, const int32_t* lens, const kivi_paging* pg) {
  if ((d->flags & KIVI_FLAG_VALUE_TOKEN_WINDOW) && (lens || pg))
    return fail(KIVI_ERR_UNSUPPORTED,
                "KIVI_FLAG_VALUE_TOKEN_WINDOW with ragged batches or paged caches is not built");
  return KIVI_OK;
}

kivi_status check_common(const kivi_dims* d, const kivi_cache* c, int32_t layer) {
  kivi_status st = check_dims(d);
  if (st != KIVI_OK) return st;
  st = check_cache(c);
  if (st != KIVI_OK) return st;
  if (layer < 0 || layer >= d->layers)
    return fail(KIVI_ERR_ARG, "layer = %d outside [0, %d)", layer, d->layers);
  return KIVI_OK;
}

kivi_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KIVI_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// A ragged batch's per-sequence counts (device int32 [B]); nullptr is accepted only
// where the caller passes no array.
kivi_status check_lens(const int32_t* lens) {
  if (!lens) return fail(KIVI_ERR_ARG, "lens is NULL");
  if ((reinterpret_cast<uintptr_t>(lens) & 3u) != 0)
    return fail(KIVI_ERR_ALIGN, "lens is not 4-byte aligned");
  return KIVI_OK;
}

// lens == nullptr: every sequence has T tokens; else sequence b has lens[b] <= T.
kivi_status quantize_common(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                            const void* x, int64_t T, int64_t ld, void* stream, bool keys,
                            const int32_t* lens = nullptr, const kivi_paging* pg = nullptr) {
  kivi_status st = check_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  st = check_paging(dims, pg);
  if (st != KIVI_OK) return st;
  st = check_vwin(dims, lens, pg);
  if (st != KIVI_OK) return st;
  if (T < 0) return fail(KIVI_ERR_ARG, "T = %lld is negative", (long long)T);
  if (T > dims->max_tokens)
    return fail(KIVI_ERR_CAPACITY, "T = %lld exceeds max_tokens = %lld", (long long)T,
                (long long)dims->max_tokens);
  if (ld < T) return fail(KIVI_ERR_ARG, "ld_tokens = %lld < T = %lld", (long long)ld, (long long)T);
  if (T == 0) return ok();
  if (!x) return fail(KIVI_ERR_ARG, "%s input is NULL", keys ? "key" : "value");
  if (!aligned16(x)) return fail(KIVI_ERR_ALIGN, "%s input is not 16-byte aligned", keys ? "key" : "value");
  const kivi::LayerView L = layer_view(dims, cache, layer, pg);
  const kivi::Lens ln{lens, T};
  hipError_t e = keys ? kivi::launch_quantize_k(L, static_cast<const __half*>(x), ld, T, ln,
                                                static_cast<hipStream_t>(stream))
                      : kivi::launch_quantize_v(L, static_cast<const __half*>(x), ld, T, ln,
                                                static_cast<hipStream_t>(stream));
  return device_status(e, keys ? "kivi_quantize_k launch" : "kivi_quantize_v launch");
}

// Checks of a decode call over T tokens; fills *L and *plan.
// check_ws false: every check but the workspace's (Lout, plan_out may then be NULL).
kivi_status decode_checks(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                          int64_t T, const void* q, float sm_scale, float* out, void* ws,
                          size_t ws_bytes, int32_t n_split, kivi::LayerView* Lout,
                          kivi::DecodePlan* plan_out, const kivi_paging* pg = nullptr,
                          bool check_ws = true) {
  kivi_status st = check_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  st = check_paging(dims, pg);
  if (st != KIVI_OK) return st;
  if (dims->group_v != dims->head_dim)
    return fail(KIVI_ERR_UNSUPPORTED, "decode requires group_v == head_dim (got %d)",
                dims->group_v);
  if (dims->group_k % 32 != 0)
    return fail(KIVI_ERR_UNSUPPORTED, "decode requires group_k in {32, 64} (got %d)",
                dims->group_k);
  if (T < 1) return fail(KIVI_ERR_ARG, "T = %lld must be >= 1", (long long)T);
  if (T > dims->max_tokens)
    return fail(KIVI_ERR_CAPACITY, "T = %lld exceeds max_tokens = %lld", (long long)T,
                (long long)dims->max_tokens);
  if (n_split < 0) return fail(KIVI_ERR_ARG, "n_split = %d is negative", n_split);
  if (!q || !out) return fail(KIVI_ERR_ARG, "q or out is NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(KIVI_ERR_ALIGN, "q or out is not 16-byte aligned");
  if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY)
    return fail(KIVI_ERR_ARG, "sm_scale is not finite");
  if (!check_ws) return KIVI_OK;
  const kivi::LayerView L = layer_view(dims, cache, layer, pg);
  const kivi::DecodePlan plan = kivi::plan_decode(L, dims->q_heads, T, n_split);
  if (!ws) return fail(KIVI_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(ws)) return fail(KIVI_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < plan.ws_total)
    return fail(KIVI_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, plan.ws_total);
  *Lout = L;
  *plan_out = plan;
  return KIVI_OK;
}

kivi_status decode_common(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                          int64_t T, const void* q, float sm_scale, float* out, void* ws,
                          size_t ws_bytes, int32_t n_split, void* stream,
                          const int32_t* lens = nullptr, const kivi_paging* pg = nullptr) {
  kivi::LayerView L;
  kivi::DecodePlan plan;
  kivi_status st = decode_checks(dims, cache, layer, T, q, sm_scale, out, ws, ws_bytes, n_split,
                                 &L, &plan, pg);
  if (st != KIVI_OK) return st;
  st = check_vwin(dims, lens, pg);
  if (st != KIVI_OK) return st;
  hipError_t e = kivi::launch_decode(L, dims->q_heads, T, static_cast<const __half*>(q), sm_scale,
                                     out, ws, plan, nullptr, kivi::Lens{lens, T},
                                     static_cast<hipStream_t>(stream));
  return device_status(e, "kivi_decode_attn launch");
}

// The fused step after its dims, cache and append checks: decode checks (which size
// the workspace), then the flush launch when the window is full and the decode launch.
kivi_status append_decode_launch(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                                 int64_t T_before, const void* k_new, const void* v_new,
                                 const void* q, float sm_scale, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const int64_t T = T_before + 1;
  kivi::LayerView L;
  kivi::DecodePlan plan;
  kivi_status st = decode_checks(dims, cache, layer, T, q, sm_scale, out, workspace,
                                 workspace_bytes, 0, &L, &plan);
  if (st != KIVI_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const __half* kn = static_cast<const __half*>(k_new);
  const __half* vn = static_cast<const __half*>(v_new);
  const kivi::AppendPlan ap = kivi::plan_append(L, T_before);
  const kivi::Lens none{nullptr, 0};
  if (ap.flush || (L.vwin && !kivi::vwin_fused_step(L, ap))) {
    // the window is full (or, with the per-token Value window, the leaving Value
    // completes a block): the append launch first, then attend
    hipError_t e = kivi::launch_append_flush(L, T_before, kn, vn, none, false, s);
    if (e != hipSuccess) return device_status(e, "kivi_append_decode flush launch");
    e = kivi::launch_decode(L, dims->q_heads, T, static_cast<const __half*>(q), sm_scale, out,
                            workspace, plan, nullptr, none, s);
    return device_status(e, "kivi_append_decode launch");
  }
  const kivi::NewRow nr{kn, vn, ap.slot, L.vwin && ap.vtok ? ap.vt : -1};
  hipError_t e = kivi::launch_decode(L, dims->q_heads, T, static_cast<const __half*>(q), sm_scale,
                                     out, workspace, plan, &nr, none, s);
  return device_status(e, "kivi_append_decode launch");
}

// ---- static decode scratch (kivi_append_decode_noalloc) ------------------------------

// The decode workspace of callers that cannot allocate device memory: one copy per GPU
// (each device that loads the library holds it until the process ends), shared by every
// kivi_append_decode_noalloc call on that GPU.  Host code never uses the array's name
// as an address: the address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zeroes n16 16-byte words (a kernel, so that a caller capturing the stream into a
// graph records a kernel node rather than a memset node).
__global__ void zero_words_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxScratchDevices];

// The current device's scratch address.  The first call on a device looks it up and
// zeroes the array on `s` (the arrival counters must start at zero; every decode leaves
// them at zero again, and each workgroup clears its own partial slot before use).
kivi_status scratch_of_current_device(void** out, hipStream_t s) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(KIVI_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(KIVI_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, s, static_cast<uint4*>(ptr),
                       kScratchBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return device_status(e, "static scratch clear launch");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return KIVI_OK;
}

// Checks of an append at T_before.
kivi_status append_checks(const kivi_dims* dims, int64_t T_before, const void* k_new,
                          const void* v_new) {
  if (T_before < 0) return fail(KIVI_ERR_ARG, "T_before = %lld is negative", (long long)T_before);
  if (T_before + 1 > dims->max_tokens)
    return fail(KIVI_ERR_CAPACITY, "T_before + 1 = %lld exceeds max_tokens = %lld",
                (long long)(T_before + 1), (long long)dims->max_tokens);
  if (!k_new || !v_new) return fail(KIVI_ERR_ARG, "k_new or v_new is NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(KIVI_ERR_ALIGN, "k_new or v_new is not 16-byte aligned");
  return KIVI_OK;
}

// ---- FP8 codec ---------------------------------------------------------------------

kivi_status check_fp8_shape(const kivi_fp8_dims* d) {
  if (!d) return fail(KIVI_ERR_ARG, "dims is NULL");
  if (d->layers < 1 || d->batch < 1 || d->kv_heads < 1 || d->q_heads < 1)
    return fail(KIVI_ERR_ARG, "layers, batch, kv_heads and q_heads must be >= 1");
  if ((int64_t)d->batch * d->kv_heads > 65535)
    return fail(KIVI_ERR_UNSUPPORTED, "batch * kv_heads = %lld exceeds 65535",
                (long long)d->batch * d->kv_heads);
  if (d->q_heads % d->kv_heads != 0)
    return fail(KIVI_ERR_ARG, "q_heads (%d) is not a multiple of kv_heads (%d)", d->q_heads,
                d->kv_heads);
  if (!is_one_of(d->q_heads / d->kv_heads, {1, 2, 4, 8}))
    return fail(KIVI_ERR_UNSUPPORTED, "q_heads / kv_heads = %d; supported: 1, 2, 4, 8",
                d->q_heads / d->kv_heads);
  if (d->head_dim != kivi::kHeadDim)
    return fail(KIVI_ERR_UNSUPPORTED, "head_dim = %d; supported: %d", d->head_dim,
                kivi::kHeadDim);
  if (d->format != KIVI_FP8_E4M3 && d->format != KIVI_FP8_E5M2)
    return fail(KIVI_ERR_UNSUPPORTED, "format = %d; supported: KIVI_FP8_E4M3, KIVI_FP8_E5M2",
                d->format);
  if (d->max_tokens < 1 || d->max_tokens % kivi::kFp8Run != 0)
    return fail(KIVI_ERR_ARG, "max_tokens = %lld must be a positive multiple of 32",
                (long long)d->max_tokens);
  return KIVI_OK;
}

// The shape rules, and one byte per channel and token: a pair's Key (or Value) codes
// must stay within the kernels' 32-bit buffer offsets.
kivi_status check_fp8_dims(const kivi_fp8_dims* d) {
  kivi_status st = check_fp8_shape(d);
  if (st != KIVI_OK) return st;
  if (d->max_tokens > kivi::kMaxPairBytes / d->head_dim)
    return fail(KIVI_ERR_UNSUPPORTED,
                "max_tokens = %lld: a pair's FP8 codes would exceed %lld bytes (at most %lld "
                "tokens)", (long long)d->max_tokens, (long long)kivi::kMaxPairBytes,
                (long long)(kivi::kMaxPairBytes / d->head_dim));
  return KIVI_OK;
}

void fp8_sizes(const kivi_fp8_dims* d, size_t out[4]) {
  const size_t unit = (size_t)d->layers * d->batch * d->kv_heads;
  out[0] = unit * (size_t)d->max_tokens * d->head_dim;
  out[1] = out[0];
  out[2] = (size_t)d->layers * d->kv_heads * sizeof(float);
  out[3] = out[2];
}

kivi_status check_fp8_common(const kivi_fp8_dims* d, const kivi_fp8_cache* c, int32_t layer) {
  kivi_status st = check_fp8_dims(d);
  if (st != KIVI_OK) return st;
  if (!c) return fail(KIVI_ERR_ARG, "cache is NULL");
  const void* p[4] = {c->k, c->v, c->k_scale, c->v_scale};
  static const char* names[4] = {"k", "v", "k_scale", "v_scale"};
  for (int i = 0; i < 4; ++i) {
    if (!p[i]) return fail(KIVI_ERR_ARG, "cache.%s is NULL", names[i]);
    if (!aligned16(p[i])) return fail(KIVI_ERR_ALIGN, "cache.%s is not 16-byte aligned", names[i]);
  }
  if (layer < 0 || layer >= d->layers)
    return fail(KIVI_ERR_ARG, "layer = %d outside [0, %d)", layer, d->layers);
  return KIVI_OK;
}

kivi::Fp8View fp8_view(const kivi_fp8_dims* d, const kivi_fp8_cache* c, int layer) {
  size_t sz[4];
  fp8_sizes(d, sz);
  const size_t Ld = (size_t)d->layers;
  kivi::Fp8View L;
  L.k = static_cast<uint8_t*>(c->k) + layer * (sz[0] / Ld);
  L.v = static_cast<uint8_t*>(c->v) + layer * (sz[1] / Ld);
  L.k_scale = static_cast<const float*>(c->k_scale) + (size_t)layer * d->kv_heads;
  L.v_scale = static_cast<const float*>(c->v_scale) + (size_t)layer * d->kv_heads;
  L.B = d->batch;
  L.H = d->kv_heads;
  L.fmt = d->format;
  L.Tmax = d->max_tokens;
  return L;
}

// ---- MXFP4 codec -------------------------------------------------------------------

kivi_status check_mx_dims(const kivi_mxfp4_dims* d) {
  if (!d) return fail(KIVI_ERR_ARG, "dims is NULL");
  if (d->reserved != 0) return fail(KIVI_ERR_ARG, "reserved = %d must be 0", d->reserved);
  const kivi_fp8_dims f{d->layers, d->batch, d->kv_heads, d->q_heads, d->head_dim, KIVI_FP8_E4M3,
                        d->max_tokens};
  kivi_status st = check_fp8_shape(&f);            // the same shape rules
  if (st != KIVI_OK) return st;
  // half a byte per channel and token: a pair's codes within 32-bit buffer offsets
  if (d->max_tokens > kivi::kMaxPairBytes / (d->head_dim / 2))
    return fail(KIVI_ERR_UNSUPPORTED,
                "max_tokens = %lld: a pair's MXFP4 codes would exceed %lld bytes (at most %lld "
                "tokens)", (long long)d->max_tokens, (long long)kivi::kMaxPairBytes,
                (long long)(kivi::kMaxPairBytes / (d->head_dim / 2)));
  return KIVI_OK;
}

void mx_sizes(const kivi_mxfp4_dims* d, size_t out[4]) {
  const size_t unit = (size_t)d->layers * d->batch * d->kv_heads * (size_t)d->max_tokens;
  out[0] = unit * (d->head_dim / 2);                 // k
  out[1] = unit * (d->head_dim / 32);                // k_scale
  out[2] = out[0];                                   // v
  out[3] = out[1];                                   // v_scale
}

kivi_status check_mx_common(const kivi_mxfp4_dims* d, const kivi_mxfp4_cache* c, int32_t layer) {
  kivi_status st = check_mx_dims(d);
  if (st != KIVI_OK) return st;
  if (!c) return fail(KIVI_ERR_ARG, "cache is NULL");
  const void* p[4] = {c->k, c->k_scale, c->v, c->v_scale};
  static const char* names[4] = {"k", "k_scale", "v", "v_scale"};
  for (int i = 0; i < 4; ++i) {
    if (!p[i]) return fail(KIVI_ERR_ARG, "cache.%s is NULL", names[i]);
    if (!aligned16(p[i])) return fail(KIVI_ERR_ALIGN, "cache.%s is not 16-byte aligned", names[i]);
  }
  if (layer < 0 || layer >= d->layers)
    return fail(KIVI_ERR_ARG, "layer = %d outside [0, %d)", layer, d->layers);
  return KIVI_OK;
}

kivi::MxView mx_view(const kivi_mxfp4_dims* d, const kivi_mxfp4_cache* c, int layer) {
  size_t sz[4];
  mx_sizes(d, sz);
  const size_t Ld = (size_t)d->layers;
  kivi::MxView L;
  L.k = static_cast<uint8_t*>(c->k) + layer * (sz[0] / Ld);
  L.k_scale = static_cast<uint8_t*>(c->k_scale) + layer * (sz[1] / Ld);
  L.v = static_cast<uint8_t*>(c->v) + layer * (sz[2] / Ld);
  L.v_scale = static_cast<uint8_t*>(c->v_scale) + layer * (sz[3] / Ld);
  L.B = d->batch;
  L.H = d->kv_heads;
  L.Tmax = d->max_tokens;
  return L;
}

}  // namespace

// The calling thread's armed kernel timer (kivi_time_next_decode).
static thread_local kivi::KernelTimer g_timer;
namespace kivi {
KernelTimer take_kernel_timer() {
  const KernelTimer t = g_timer;
  g_timer = KernelTimer{};
  return t;
}
}  // namespace kivi

extern "C" {

kivi_status kivi_mxfp4_cache_sizes(const kivi_mxfp4_dims* dims, size_t bytes[4]) {
  kivi_status st = check_mx_dims(dims);
  if (st != KIVI_OK) return st;
  if (!bytes) return fail(KIVI_ERR_ARG, "bytes is NULL");
  mx_sizes(dims, bytes);
  return ok();
}

kivi_status kivi_mxfp4_quantize(const kivi_mxfp4_dims* dims, const kivi_mxfp4_cache* cache,
                                int32_t layer, const void* k, const void* v, int64_t T,
                                int64_t ld_tokens, void* stream) {
  kivi_status st = check_mx_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  if (T < 0) return fail(KIVI_ERR_ARG, "T = %lld is negative", (long long)T);
  if (T > dims->max_tokens)
    return fail(KIVI_ERR_CAPACITY, "T = %lld exceeds max_tokens = %lld", (long long)T,
                (long long)dims->max_tokens);
  if (ld_tokens < T)
    return fail(KIVI_ERR_ARG, "ld_tokens = %lld < T = %lld", (long long)ld_tokens, (long long)T);
  if (T == 0) return ok();
  if (!k || !v) return fail(KIVI_ERR_ARG, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(KIVI_ERR_ALIGN, "k or v is not 16-byte aligned");
  hipError_t e = kivi::launch_mx_quantize(mx_view(dims, cache, layer), static_cast<const __half*>(k),
                                          static_cast<const __half*>(v), ld_tokens, T,
                                          static_cast<hipStream_t>(stream));
  return device_status(e, "kivi_mxfp4_quantize launch");
}

kivi_status kivi_mxfp4_append(const kivi_mxfp4_dims* dims, const kivi_mxfp4_cache* cache,
                              int32_t layer, int64_t T_before, const void* k_new,
                              const void* v_new, void* stream) {
  kivi_status st = check_mx_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  if (T_before < 0) return fail(KIVI_ERR_ARG, "T_before = %lld is negative", (long long)T_before);
  if (T_before + 1 > dims->max_tokens)
    return fail(KIVI_ERR_CAPACITY, "T_before + 1 = %lld exceeds max_tokens = %lld",
                (long long)(T_before + 1), (long long)dims->max_tokens);
  if (!k_new || !v_new) return fail(KIVI_ERR_ARG, "k_new or v_new is NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(KIVI_ERR_ALIGN, "k_new or v_new is not 16-byte aligned");
  hipError_t e = kivi::launch_mx_append(mx_view(dims, cache, layer),
                                        static_cast<const __half*>(k_new),
                                        static_cast<const __half*>(v_new), T_before,
                                        static_cast<hipStream_t>(stream));
  return device_status(e, "kivi_mxfp4_append launch");
}

kivi_status kivi_mxfp4_decode_workspace_bytes(const kivi_mxfp4_dims* dims, int64_t T,
                                              int32_t n_split, size_t* bytes) {
  kivi_status st = check_mx_dims(dims);
  if (st != KIVI_OK) return st;
  if (!bytes) return fail(KIVI_ERR_ARG, "bytes is NULL");
  if (T < 1 || T > dims->max_tokens)
    return fail(T < 1 ? KIVI_ERR_ARG : KIVI_ERR_CAPACITY, "T = %lld outside [1, max_tokens]",
                (long long)T);
  if (n_split < 0) return fail(KIVI_ERR_ARG, "n_split = %d is negative", n_split);
  *bytes = kivi::plan_fp8_decode(dims->batch, dims->kv_heads, dims->q_heads, T, n_split).ws_total;
  return ok();
}

}  // extern "C"

namespace {

kivi_status mx_decode_common(const kivi_mxfp4_dims* dims, const kivi_mxfp4_cache* cache,
                             int32_t layer, int64_t T, const void* q, float sm_scale, float* out,
                             void* workspace, size_t workspace_bytes, int32_t n_split,
                             const void* k_new, const void* v_new, void* stream) {
  kivi_status st = check_mx_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  if (T < 1) return fail(KIVI_ERR_ARG, "T = %lld must be >= 1", (long long)T);
  if (T > dims->max_tokens)
    return fail(KIVI_ERR_CAPACITY, "T = %lld exceeds max_tokens = %lld", (long long)T,
                (long long)dims->max_tokens);
  if (n_split < 0) return fail(KIVI_ERR_ARG, "n_split = %d is negative", n_split);
  if (!q || !out) return fail(KIVI_ERR_ARG, "q or out is NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(KIVI_ERR_ALIGN, "q or out is not 16-byte aligned");
  if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY)
    return fail(KIVI_ERR_ARG, "sm_scale is not finite");
  const kivi::Fp8Plan plan =
      kivi::plan_fp8_decode(dims->batch, dims->kv_heads, dims->q_heads, T, n_split);
  if (!workspace) return fail(KIVI_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(KIVI_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < plan.ws_total)
    return fail(KIVI_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                plan.ws_total);
  hipError_t e = kivi::launch_mx_decode(mx_view(dims, cache, layer), dims->q_heads, T,
                                        static_cast<const __half*>(q), sm_scale, out, workspace,
                                        plan, static_cast<const __half*>(k_new),
                                        static_cast<const __half*>(v_new),
                                        static_cast<hipStream_t>(stream));
  return device_status(e, "kivi_mxfp4 decode launch");
}

}  // namespace

extern "C" {

kivi_status kivi_mxfp4_decode_attn(const kivi_mxfp4_dims* dims, const kivi_mxfp4_cache* cache,
                                   int32_t layer, int64_t T, const void* q, float sm_scale,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   int32_t n_split, void* stream) {
  return mx_decode_common(dims, cache, layer, T, q, sm_scale, out, workspace, workspace_bytes,
                          n_split, nullptr, nullptr, stream);
}

kivi_status kivi_mxfp4_append_decode(const kivi_mxfp4_dims* dims, const kivi_mxfp4_cache* cache,
                                     int32_t layer, int64_t T_before, const void* k_new,
                                     const void* v_new, const void* q, float sm_scale,
                                     float* out, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  kivi_status st = check_mx_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  if (T_before < 0) return fail(KIVI_ERR_ARG, "T_before = %lld is negative", (long long)T_before);
  if (T_before + 1 > dims->max_tokens)
    return fail(KIVI_ERR_CAPACITY, "T_before + 1 = %lld exceeds max_tokens = %lld",
                (long long)(T_before + 1), (long long)dims->max_tokens);
  if (!k_new || !v_new) return fail(KIVI_ERR_ARG, "k_new or v_new is NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(KIVI_ERR_ALIGN, "k_new or v_new is not 16-byte aligned");
  return mx_decode_common(dims, cache, layer, T_before + 1, q, sm_scale, out, workspace,
                          workspace_bytes, 0, k_new, v_new, stream);
}

kivi_status kivi_fp8_cache_sizes(const kivi_fp8_dims* dims, size_t bytes[4]) {
  kivi_status st = check_fp8_dims(dims);
  if (st != KIVI_OK) return st;
  if (!bytes) return fail(KIVI_ERR_ARG, "bytes is NULL");
  fp8_sizes(dims, bytes);
  return ok();
}

kivi_status kivi_fp8_quantize(const kivi_fp8_dims* dims, const kivi_fp8_cache* cache,
                              int32_t layer, const void* k, const void* v, int64_t T,
                              int64_t ld_tokens, void* stream) {
  kivi_status st = check_fp8_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  if (T < 0) return fail(KIVI_ERR_ARG, "T = %lld is negative", (long long)T);
  if (T > dims->max_tokens)
    return fail(KIVI_ERR_CAPACITY, "T = %lld exceeds max_tokens = %lld", (long long)T,
                (long long)dims->max_tokens);
  if (ld_tokens < T)
    return fail(KIVI_ERR_ARG, "ld_tokens = %lld < T = %lld", (long long)ld_tokens, (long long)T);
  if (T == 0) return ok();
  if (!k || !v) return fail(KIVI_ERR_ARG, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(KIVI_ERR_ALIGN, "k or v is not 16-byte aligned");
  hipError_t e = kivi::launch_fp8_quantize(fp8_view(dims, cache, layer), static_cast<const __half*>(k),
                                           static_cast<const __half*>(v), ld_tokens, T,
                                           static_cast<hipStream_t>(stream));
  return device_status(e, "kivi_fp8_quantize launch");
}

kivi_status kivi_fp8_append(const kivi_fp8_dims* dims, const kivi_fp8_cache* cache, int32_t layer,
                            int64_t T_before, const void* k_new, const void* v_new, void* stream) {
  kivi_status st = check_fp8_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  if (T_before < 0) return fail(KIVI_ERR_ARG, "T_before = %lld is negative", (long long)T_before);
  if (T_before + 1 > dims->max_tokens)
    return fail(KIVI_ERR_CAPACITY, "T_before + 1 = %lld exceeds max_tokens = %lld",
                (long long)(T_before + 1), (long long)dims->max_tokens);
  if (!k_new || !v_new) return fail(KIVI_ERR_ARG, "k_new or v_new is NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(KIVI_ERR_ALIGN, "k_new or v_new is not 16-byte aligned");
  hipError_t e = kivi::launch_fp8_append(fp8_view(dims, cache, layer),
                                         static_cast<const __half*>(k_new),
                                         static_cast<const __half*>(v_new), T_before,
                                         static_cast<hipStream_t>(stream));
  return device_status(e, "kivi_fp8_append launch");
}

kivi_status kivi_fp8_decode_workspace_bytes(const kivi_fp8_dims* dims, int64_t T, int32_t n_split,
                                            size_t* bytes) {
  kivi_status st = check_fp8_dims(dims);
  if (st != KIVI_OK) return st;
  if (!bytes) return fail(KIVI_ERR_ARG, "bytes is NULL");
  if (T < 1 || T > dims->max_tokens)
    return fail(T < 1 ? KIVI_ERR_ARG : KIVI_ERR_CAPACITY, "T = %lld outside [1, max_tokens]",
                (long long)T);
  if (n_split < 0) return fail(KIVI_ERR_ARG, "n_split = %d is negative", n_split);
  *bytes = kivi::plan_fp8_decode(dims->batch, dims->kv_heads, dims->q_heads, T, n_split).ws_total;
  return ok();
}

kivi_status kivi_fp8_decode_attn(const kivi_fp8_dims* dims, const kivi_fp8_cache* cache,
                                 int32_t layer, int64_t T, const void* q, float sm_scale,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 int32_t n_split, void* stream) {
  kivi_status st = check_fp8_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  if (T < 1) return fail(KIVI_ERR_ARG, "T = %lld must be >= 1", (long long)T);
  if (T > dims->max_tokens)
    return fail(KIVI_ERR_CAPACITY, "T = %lld exceeds max_tokens = %lld", (long long)T,
                (long long)dims->max_tokens);
  if (n_split < 0) return fail(KIVI_ERR_ARG, "n_split = %d is negative", n_split);
  if (!q || !out) return fail(KIVI_ERR_ARG, "q or out is NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(KIVI_ERR_ALIGN, "q or out is not 16-byte aligned");
  if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY)
    return fail(KIVI_ERR_ARG, "sm_scale is not finite");
  const kivi::Fp8Plan plan =
      kivi::plan_fp8_decode(dims->batch, dims->kv_heads, dims->q_heads, T, n_split);
  if (!workspace) return fail(KIVI_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(KIVI_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < plan.ws_total)
    return fail(KIVI_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                plan.ws_total);
  hipError_t e = kivi::launch_fp8_decode(fp8_view(dims, cache, layer), dims->q_heads, T,
                                         static_cast<const __half*>(q), sm_scale, out, workspace,
                                         plan, static_cast<hipStream_t>(stream));
  return device_status(e, "kivi_fp8_decode_attn launch");
}


kivi_status kivi_cache_sizes(const kivi_dims* dims, size_t bytes[KIVI_NUM_BUFFERS]) {
  kivi_status st = check_dims(dims);
  if (st != KIVI_OK) return st;
  if (!bytes) return fail(KIVI_ERR_ARG, "bytes is NULL");
  buffer_sizes(dims, nullptr, bytes);
  return ok();
}

kivi_status kivi_paged_cache_sizes(const kivi_dims* dims, const kivi_paging* paging,
                                   size_t bytes[KIVI_NUM_BUFFERS]) {
  kivi_status st = check_dims(dims);
  if (st != KIVI_OK) return st;
  if (!paging) return fail(KIVI_ERR_ARG, "paging is NULL");
  if (!bytes) return fail(KIVI_ERR_ARG, "bytes is NULL");
  st = check_page_geometry(dims, paging);          // the table is not needed for sizes
  if (st != KIVI_OK) return st;
  buffer_sizes(dims, paging, bytes);
  return ok();
}

kivi_status kivi_quantize_k(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                            const void* k, int64_t T, int64_t ld_tokens, void* stream) {
  return quantize_common(dims, cache, layer, k, T, ld_tokens, stream, true);
}

kivi_status kivi_quantize_v(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                            const void* v, int64_t T, int64_t ld_tokens, void* stream) {
  return quantize_common(dims, cache, layer, v, T, ld_tokens, stream, false);
}

kivi_status append_common(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                          int64_t T_before, const void* k_new, const void* v_new, void* stream,
                          const int32_t* lens, const kivi_paging* pg = nullptr) {
  kivi_status st = check_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  st = check_paging(dims, pg);
  if (st != KIVI_OK) return st;
  st = check_vwin(dims, lens, pg);
  if (st != KIVI_OK) return st;
  st = append_checks(dims, T_before, k_new, v_new);
  if (st != KIVI_OK) return st;
  const kivi::LayerView L = layer_view(dims, cache, layer, pg);
  hipError_t e = kivi::launch_append_flush(L, T_before, static_cast<const __half*>(k_new),
                                           static_cast<const __half*>(v_new),
                                           kivi::Lens{lens, T_before}, false,
                                           static_cast<hipStream_t>(stream));
  return device_status(e, "kivi_append_flush launch");
}

kivi_status kivi_append_flush(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                              int64_t T_before, const void* k_new, const void* v_new,
                              void* stream) {
  return append_common(dims, cache, layer, T_before, k_new, v_new, stream, nullptr);
}

kivi_status kivi_decode_workspace_bytes_split(const kivi_dims* dims, int64_t T, int32_t n_split,
                                              size_t* bytes) {
  kivi_status st = check_dims(dims);
  if (st != KIVI_OK) return st;
  if (!bytes) return fail(KIVI_ERR_ARG, "bytes is NULL");
  if (T < 1 || T > dims->max_tokens)
    return fail(T < 1 ? KIVI_ERR_ARG : KIVI_ERR_CAPACITY, "T = %lld outside [1, max_tokens]",
                (long long)T);
  if (n_split < 0) return fail(KIVI_ERR_ARG, "n_split = %d is negative", n_split);
  const kivi::LayerView L = shape_view(dims);
  *bytes = kivi::plan_decode(L, dims->q_heads, T, n_split).ws_total;
  return ok();
}

kivi_status kivi_decode_workspace_bytes(const kivi_dims* dims, int64_t T, size_t* bytes) {
  return kivi_decode_workspace_bytes_split(dims, T, 0, bytes);
}

kivi_status kivi_decode_splits(const kivi_dims* dims, int64_t T, int32_t* n_split) {
  kivi_status st = check_dims(dims);
  if (st != KIVI_OK) return st;
  if (!n_split) return fail(KIVI_ERR_ARG, "n_split is NULL");
  if (T < 1 || T > dims->max_tokens)
    return fail(T < 1 ? KIVI_ERR_ARG : KIVI_ERR_CAPACITY, "T = %lld outside [1, max_tokens]",
                (long long)T);
  const kivi::LayerView L = shape_view(dims);
  *n_split = kivi::plan_decode(L, dims->q_heads, T, 0).n_split;
  return ok();
}

kivi_status kivi_decode_attn(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                             int64_t T, const void* q, float sm_scale, float* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(dims, cache, layer, T, q, sm_scale, out, workspace, workspace_bytes, 0,
                       stream);
}

kivi_status kivi_decode_attn_split(const kivi_dims* dims, const kivi_cache* cache,
                                   int32_t layer, int64_t T, const void* q, float sm_scale,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   int32_t n_split, void* stream) {
  return decode_common(dims, cache, layer, T, q, sm_scale, out, workspace, workspace_bytes,
                       n_split, stream);
}

kivi_status kivi_append_decode(const kivi_dims* dims, const kivi_cache* cache, int32_t layer,
                               int64_t T_before, const void* k_new, const void* v_new,
                               const void* q, float sm_scale, float* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  kivi_status st = check_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  st = append_checks(dims, T_before, k_new, v_new);
  if (st != KIVI_OK) return st;
  return append_decode_launch(dims, cache, layer, T_before, k_new, v_new, q, sm_scale, out,
                              workspace, workspace_bytes, stream);
}

kivi_status kivi_append_decode_noalloc(const kivi_dims* dims, const kivi_cache* cache,
                                       int32_t layer, int64_t T_before, const void* k_new,
                                       const void* v_new, const void* q, float sm_scale,
                                       float* out, void* stream) {
  kivi_status st = check_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  st = append_checks(dims, T_before, k_new, v_new);
  if (st != KIVI_OK) return st;
  st = decode_checks(dims, cache, layer, T_before + 1, q, sm_scale, out, nullptr, 0, 0, nullptr,
                     nullptr, nullptr, /*check_ws=*/false);
  if (st != KIVI_OK) return st;
  const kivi::DecodePlan plan =
      kivi::plan_decode(shape_view(dims), dims->q_heads, T_before + 1, 0);
  if (plan.ws_total > kScratchBytes)
    return fail(KIVI_ERR_UNSUPPORTED,
                "this step needs %zu bytes of decode scratch; the library's static scratch "
                "holds %zu (use kivi_append_decode with a workspace)",
                plan.ws_total, kScratchBytes);
  void* ws = nullptr;
  st = scratch_of_current_device(&ws, static_cast<hipStream_t>(stream));
  if (st != KIVI_OK) return st;
  return append_decode_launch(dims, cache, layer, T_before, k_new, v_new, q, sm_scale, out, ws,
                              kScratchBytes, stream);
}

// ---- ragged batches ------------------------------------------------------------------

kivi_status kivi_quantize_k_varlen(const kivi_dims* dims, const kivi_cache* cache,
                                   const kivi_paging* paging, int32_t layer, const void* k,
                                   const int32_t* lens, int64_t T_hi, int64_t ld_tokens,
                                   void* stream) {
  kivi_status st = check_lens(lens);
  if (st != KIVI_OK) return st;
  return quantize_common(dims, cache, layer, k, T_hi, ld_tokens, stream, true, lens, paging);
}

kivi_status kivi_quantize_v_varlen(const kivi_dims* dims, const kivi_cache* cache,
                                   const kivi_paging* paging, int32_t layer, const void* v,
                                   const int32_t* lens, int64_t T_hi, int64_t ld_tokens,
                                   void* stream) {
  kivi_status st = check_lens(lens);
  if (st != KIVI_OK) return st;
  return quantize_common(dims, cache, layer, v, T_hi, ld_tokens, stream, false, lens, paging);
}

kivi_status kivi_append_flush_varlen(const kivi_dims* dims, const kivi_cache* cache,
                                     const kivi_paging* paging, int32_t layer,
                                     const int32_t* T_before, int64_t T_hi, const void* k_new,
                                     const void* v_new, void* stream) {
  kivi_status st = check_lens(T_before);
  if (st != KIVI_OK) return st;
  return append_common(dims, cache, layer, T_hi, k_new, v_new, stream, T_before, paging);
}

kivi_status kivi_decode_attn_varlen(const kivi_dims* dims, const kivi_cache* cache,
                                    const kivi_paging* paging, int32_t layer,
                                    const int32_t* lens, int64_t T_hi, const void* q,
                                    float sm_scale, float* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  kivi_status st = check_lens(lens);
  if (st != KIVI_OK) return st;
  return decode_common(dims, cache, layer, T_hi, q, sm_scale, out, workspace, workspace_bytes,
                       0, stream, lens, paging);
}

}  // extern "C"

namespace {

// The ragged decode step.  host_lens, when given, is a host copy of T_before: a step in
// which no sequence's window is full skips the flush launch, which would do nothing.
kivi_status append_decode_varlen(const kivi_dims* dims, const kivi_cache* cache,
                                 const kivi_paging* paging, int32_t layer, const int32_t* T_before,
                                 const int32_t* host_lens, int64_t T_hi, const void* k_new,
                                 const void* v_new, const void* q, float sm_scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  kivi_status st = check_lens(T_before);
  if (st != KIVI_OK) return st;
  st = check_common(dims, cache, layer);
  if (st != KIVI_OK) return st;
  st = check_vwin(dims, T_before, paging);
  if (st != KIVI_OK) return st;
  st = append_checks(dims, T_hi, k_new, v_new);
  if (st != KIVI_OK) return st;
  kivi::LayerView L;
  kivi::DecodePlan plan;
  st = decode_checks(dims, cache, layer, T_hi + 1, q, sm_scale, out, workspace, workspace_bytes,
                     0, &L, &plan, paging);
  if (st != KIVI_OK) return st;
  bool flush_launch = true;
  if (host_lens) {
    flush_launch = false;
    for (int b = 0; b < dims->batch; ++b) {
      if (host_lens[b] < 0 || host_lens[b] > T_hi)
        return fail(KIVI_ERR_ARG, "T_before_host entry outside [0, T_hi]");
      if (kivi::plan_append(L, host_lens[b]).flush) flush_launch = true;
    }
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const __half* kn = static_cast<const __half*>(k_new);
  const __half* vn = static_cast<const __half*>(v_new);
  const kivi::Lens ln{T_before, T_hi};
  // the sequences whose window is full flush first (the others' blocks return at once);
  // the decode launch then stores every new row and attends
  if (flush_launch) {
    const hipError_t e = kivi::launch_append_flush(L, T_hi, kn, vn, ln, true, s);
    if (e != hipSuccess) return device_status(e, "kivi_append_decode_varlen flush launch");
  }
  const kivi::NewRow nr{kn, vn, kivi::plan_append(L, T_hi).slot};
  const hipError_t e = kivi::launch_decode(L, dims->q_heads, T_hi + 1,
                                           static_cast<const __half*>(q), sm_scale, out,
                                           workspace, plan, &nr, ln, s);
  return device_status(e, "kivi_append_decode_varlen launch");
}

}  // namespace

extern "C" {

kivi_status kivi_append_decode_varlen(const kivi_dims* dims, const kivi_cache* cache,
                                      const kivi_paging* paging, int32_t layer,
                                      const int32_t* T_before, int64_t T_hi, const void* k_new,
                                      const void* v_new, const void* q, float sm_scale,
                                      float* out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return append_decode_varlen(dims, cache, paging, layer, T_before, nullptr, T_hi, k_new, v_new,
                              q, sm_scale, out, workspace, workspace_bytes, stream);
}

kivi_status kivi_append_decode_varlen_host(const kivi_dims* dims, const kivi_cache* cache,
                                           const kivi_paging* paging, int32_t layer,
                                           const int32_t* T_before,
                                           const int32_t* T_before_host, int64_t T_hi,
                                           const void* k_new, const void* v_new, const void* q,
                                           float sm_scale, float* out, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (!T_before_host) return fail(KIVI_ERR_ARG, "T_before_host is NULL");
  return append_decode_varlen(dims, cache, paging, layer, T_before, T_before_host, T_hi, k_new,
                              v_new, q, sm_scale, out, workspace, workspace_bytes, stream);
}

const char* kivi_last_error(void) { return g_err; }

// ---- measurement aid ----------------------------------------------------------------

kivi_status kivi_time_next_decode(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(KIVI_ERR_ARG, "start_event and stop_event must both be set or both be null");
  g_timer.start = static_cast<hipEvent_t>(start_event);
  g_timer.stop = static_cast<hipEvent_t>(stop_event);
  return KIVI_OK;
}

int32_t kivi_abi_version(void) { return 9; }

}  // extern "C"
