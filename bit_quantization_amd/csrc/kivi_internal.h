// Internal declarations shared by the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kivi {

constexpr int kHeadDim = 128;   // head_dim this build's kernels are written for
constexpr int kVRun = 16;       // tokens per packed Value run
// Largest buffer of one (sequence, KV head) pair the kernels address: their buffer
// offsets are 32-bit.
constexpr int64_t kMaxPairBytes = 0x7FFFFF00;

// Compute units of the current device (cached per device); 256, one MI355X's, when no
// device can be queried (planning on a host without a GPU).
int device_cus();

// Device pointers of one layer, already offset to that layer, plus the dims.  The
// history buffers hold one section per (b, h) pair of Tmax tokens, or, for a paged
// cache, one section per KV head: a pool of `pages` pages of P = 2^page_log2 tokens,
// table[b * pages_per_seq + i] naming the page of sequence b's history tokens
// [iP, (i+1)P).
struct LayerView {
  uint8_t* k_codes;   // [sections][rows][d*b/8]
  __half* k_scale;    // [sections][rows/G][d]
  __half* k_zero;
  uint8_t* v_codes;   // [sections][rows/16][d][16*b/8]
  __half* v_scale;    // [sections][rows][d/Gv]
  __half* v_zero;
  __half* k_resid;    // [B][H][S + R][d]: rows [0, S) the sink tokens, then the window
  __half* v_resid;
  float* scale_max;   // [B][H][2]: largest Key scale, largest Value scale
  int B, H, d, bits, G, Gv, R;
  int S;              // sink tokens kept in float16 (tokens [0, S) of each sequence)
  int aging;          // 0: a full window is flushed whole; 1: only its oldest Key group
  int vwin;           // 1: the per-token Value window (Values leave it one at a time)
  int det;            // 1: deterministic decode (fixed block order in every wave)
  int64_t Tmax;
  const int32_t* table;   // nullptr: contiguous history, one section per pair
  int page_log2;
  int pages_per_seq;
  int64_t pages;

  // Tokens of one history section, the section of a (b, h) pair, and where history
  // token t of sequence b sits in its section (a page-table entry outside [0, pages)
  // is clamped, so every access stays inside the pool).
  __host__ __device__ int64_t rows() const { return table ? pages << page_log2 : Tmax; }
  __host__ __device__ int64_t section(int64_t pair) const { return table ? pair % H : pair; }
  __device__ int64_t hist_token(int64_t b, int64_t t) const {
    if (!table) return t;
    int64_t pg = table[b * pages_per_seq + (t >> page_log2)];
    pg = pg < 0 ? 0 : pg >= pages ? pages - 1 : pg;
    return (pg << page_log2) + (t & ((int64_t(1) << page_log2) - 1));
  }

  // Per-section element strides of each history buffer; per-pair of the window.
  __host__ __device__ int64_t kc_pair() const { return rows() * (d * bits / 8); }
  __host__ __device__ int64_t ks_pair() const { return (rows() / G) * d; }
  __host__ __device__ int64_t vc_pair() const { return rows() * (d * bits / 8); }
  __host__ __device__ int64_t vs_pair() const { return rows() * (d / Gv); }
  __host__ __device__ int64_t rs_pair() const { return (int64_t)(S + R) * d; }
};

// Window tokens after Tk tokens (those after the sink): the full window flushes
// whole, so r = ((Tk - 1) mod R) + 1; with group aging only its oldest G tokens
// leave, so r = Tk up to R and R - G + ((Tk - R - 1) mod G) + 1 after.
__host__ __device__ inline int64_t window_len(int64_t Tk, int R, int G, int aging) {
  if (Tk == 0) return 0;
  if (!aging) return (Tk - 1) % R + 1;
  return Tk <= R ? Tk : R - G + (Tk - R - 1) % G + 1;
}

// T cached tokens with S sink tokens: the first min(T, S) stay in float16 (residual
// rows [0, S)); the rest follow the window rules counted from S: Tq of them are in
// the quantized history, r in the window.  The window is a ring over residual rows
// [S, S + R): token i after the sink sits in row S + (i mod R), so its r tokens
// start at row S + ring and wrap after row S + R - 1 (ring = Tq mod R, a multiple
// of G; 0 when the full window flushes).
//
// With the per-token Value window (L.vwin) Values follow their own rule: the Value
// window holds the rv = min(Tk, R) most recent tokens after the sink, in the same ring
// rows (token i in row S + (i mod R)), and the Tqv = Tk - rv tokens before them are the
// quantized Value history.  Tqv <= Tq: tokens [Tqv, Tq) have quantized Keys and float16
// Values.  Without it Tqv = Tq and rv = r.
struct TokenSplit {
  int64_t ns, Tq, r;
  int ring;
  int64_t Tqv, rv;
  int ring_v;
  __host__ __device__ int64_t fp16_rows() const { return ns + r; }   // sink rows and window tokens
};
__host__ __device__ inline TokenSplit split_tokens(const LayerView& L, int64_t T) {
  TokenSplit t;
  t.ns = T < L.S ? T : L.S;
  const int64_t Tk = T - t.ns;
  t.r = window_len(Tk, L.R, L.G, L.aging);
  t.Tq = Tk - t.r;
  t.ring = (int)(t.Tq % L.R);
  t.Tqv = L.vwin ? (Tk > L.R ? Tk - L.R : 0) : t.Tq;
  t.rv = Tk - t.Tqv;
  t.ring_v = (int)(t.Tqv % L.R);
  return t;
}

// Where an appended token goes: the sink row T_before while the sink fills; else its
// ring row in the window, after flushing the oldest n window tokens (rows
// [first, first + n), never wrapping) into the history at token t0 when the window
// is full.  The new token then takes row `first`.
// With the per-token Value window the flush moves Keys only; instead, once the Value
// window is full (Tk >= R), its oldest token — in row `slot`, which the new token takes —
// is quantized on its own into Value history token vt (vtok).
struct AppendPlan {
  int flush;      // 1: quantize n window tokens into the history first
  int n;          // tokens flushed: R, or G with group aging
  int first;      // residual row of the oldest window token (flush only)
  int slot;       // residual row of the new token
  int64_t t0;     // history token of the oldest window token (flush only)
  int vtok;       // 1: quantize the Value in row `slot` into history token vt first
  int64_t vt;
};
__host__ __device__ inline AppendPlan plan_append(const LayerView& L, int64_t T_before) {
  if (T_before < L.S) return AppendPlan{0, 0, 0, (int)T_before, 0, 0, 0};
  const int64_t Tk = T_before - L.S;
  const int64_t r = window_len(Tk, L.R, L.G, L.aging);
  const int slot = L.S + (int)(Tk % L.R);
  const int vtok = L.vwin && Tk >= L.R;
  const int64_t vt = vtok ? Tk - L.R : 0;
  if (r < L.R) return AppendPlan{0, 0, 0, slot, 0, vtok, vt};
  const int64_t Tq = Tk - r;
  return AppendPlan{1, L.aging ? L.G : L.R, L.S + (int)(Tq % L.R), slot, Tq, vtok, vt};
}

// Tokens per block of the decode's quantized-history loop.
constexpr int kDecodeBlockTokens = 64;
// A step of the per-token Value window that flushes no Key group runs as one decode
// launch (the decode quantizes the leaving Value), unless that Value completes a block
// of the quantized-history loop: the block's codes are then read by other workgroups of
// the same launch, so they are written by an append launch first.
__host__ __device__ inline bool vwin_fused_step(const LayerView& L, const AppendPlan& ap) {
  return L.vwin && !ap.flush && (!ap.vtok || (ap.vt + 1) % kDecodeBlockTokens != 0);
}

// Per-sequence token counts of a ragged batch: device int32 [B] holding T_b (or T_b
// - 1 for a decode step that appends), clamped on the device into [lo, hi] so that
// every access stays inside the cache whatever the array holds.
struct Lens {
  const int32_t* p;     // nullptr: every sequence has the call's uniform T
  int64_t hi;           // upper bound the launch was planned for
  __device__ int64_t get(int64_t b, int64_t lo) const {
    const int64_t t = p[b];
    return t < lo ? lo : t > hi ? hi : t;
  }
};

// ---- launchers (return hipGetLastError() of the launch) -------------------------

// Prefill of T tokens of src ([B][H][ld][d]): the sink tokens to residual rows
// [0, ns), the history tokens [S, S + Tq) quantized, the last r to their ring rows.
// With lens.p set, sequence b has lens.get(b, 0) tokens and T is lens.hi.
hipError_t launch_quantize_k(const LayerView& L, const __half* src, int64_t ld, int64_t T,
                             Lens lens, hipStream_t s);
hipError_t launch_quantize_v(const LayerView& L, const __half* src, int64_t ld, int64_t T,
                             Lens lens, hipStream_t s);

// Append one row; when the window is full, flush its oldest tokens first (plan_append).
// With lens.p set, sequence b appends at T_before = lens.get(b, 0) (T_before is
// lens.hi), and flush_only leaves the new row of a sequence that does not flush to the
// decode launch that follows.
hipError_t launch_append_flush(const LayerView& L, int64_t T_before, const __half* k_new,
                               const __half* v_new, Lens lens, bool flush_only,
                               hipStream_t s);

// Decode attention: split-K partials + fixed-order merge.
struct DecodePlan {
  int n_split;          // token splits per (b, kv head)
  int64_t n_groups;     // quantized Key groups per (b, kv head)
  int r;                // float16 tokens: sink rows and window
  int ring;             // window ring start (split_tokens)
  int64_t tq_blocks;    // tokens the 64-token blocks cover
  int n_mix;            // 32-row chunks of quantized Keys past them (per-token Value window)
  size_t ws_partials;   // bytes of partial results
  size_t ws_counters;   // bytes of per-pair arrival counters
  size_t ws_total;
};
DecodePlan plan_decode(const LayerView& L, int q_heads, int64_t T, int n_split_req);
// A token appended by the decode launch itself: its rows are read from k/v (float16
// [B][H_kv][d]) as window row `slot`, and the launch also stores them there.
// Measurement aid (kivi_time_next_decode): a pair of events that the calling thread's
// next decode-kernel launch records at the kernel's own start and end.
struct KernelTimer {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
KernelTimer take_kernel_timer();   // the armed pair (or none); disarms
// Launches a decode kernel as hipLaunchKernelGGL does, or, with a timer armed, through
// hipExtLaunchKernel with the timer's events.
template <typename K, typename... Args>
void launch_decode_kernel(K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  const KernelTimer t = take_kernel_timer();
  if (t.start)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t.start, t.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

struct NewRow {
  const __half* k;
  const __half* v;
  int slot;
  int64_t vt = -1;      // per-token Value window: history token whose Value leaves the
                        // window in this step (its row is slot), quantized by the decode
};
// With lens.p set, sequence b attends over lens.get(b, 1) tokens (T = lens.hi), or,
// with new_row set, appends at T_before = lens.get(b, 0) and attends over T_before + 1
// (T = lens.hi + 1); new_row->slot is then found per sequence.
hipError_t launch_decode(const LayerView& L, int q_heads, int64_t T, const __half* q,
                         float sm_scale, float* out, void* ws, const DecodePlan& plan,
                         const NewRow* new_row, Lens lens, hipStream_t s);

// ---- FP8 KV codec -----------------------------------------------------------------
// One layer of an FP8 cache: Key codes [B][H][Tmax][d], Value codes in 32-token runs
// [B][H][Tmax/32][d][32], float32 scales per KV head.
constexpr int kFp8Run = 32;
struct Fp8View {
  uint8_t* k;
  uint8_t* v;
  const float* k_scale;   // [H]
  const float* v_scale;   // [H]
  int B, H, fmt;          // fmt: 0 E4M3, 1 E5M2
  int64_t Tmax;
  __host__ __device__ int64_t pair_bytes() const { return Tmax * kHeadDim; }
};
struct Fp8Plan {
  int n_split;            // workgroups per (sequence, KV head)
  size_t ws_counters, ws_partials, ws_total;
};
hipError_t launch_fp8_quantize(const Fp8View& L, const __half* k, const __half* v, int64_t ld,
                               int64_t T, hipStream_t s);
hipError_t launch_fp8_append(const Fp8View& L, const __half* k_new, const __half* v_new,
                             int64_t t, hipStream_t s);
Fp8Plan plan_fp8_decode(int B, int H, int q_heads, int64_t T, int n_split_req);
hipError_t launch_fp8_decode(const Fp8View& L, int q_heads, int64_t T, const __half* q,
                             float sm_scale, float* out, void* ws, const Fp8Plan& plan,
                             hipStream_t s);

// ---- MXFP4 KV codec ---------------------------------------------------------------
// One layer of an MXFP4 cache, per (sequence, KV head): Key codes [Tmax][d/2] bytes and
// scales [Tmax][d/32]; Value codes in 32-token runs [Tmax/32][d][16] bytes and scales
// [Tmax/32][d/32][32] (E8M0 codes).
struct MxView {
  uint8_t* k;
  uint8_t* k_scale;
  uint8_t* v;
  uint8_t* v_scale;
  int B, H;
  int64_t Tmax;
  __host__ __device__ int64_t k_pair() const { return Tmax * (kHeadDim / 2); }
  __host__ __device__ int64_t ks_pair() const { return Tmax * (kHeadDim / 32); }
  __host__ __device__ int64_t v_pair() const { return Tmax * (kHeadDim / 2); }
  __host__ __device__ int64_t vs_pair() const { return Tmax * (kHeadDim / 32); }
};
hipError_t launch_mx_quantize(const MxView& L, const __half* k, const __half* v, int64_t ld,
                              int64_t T, hipStream_t s);
hipError_t launch_mx_append(const MxView& L, const __half* k_new, const __half* v_new, int64_t t,
                            hipStream_t s);
// Planned as the FP8 decode (32-token blocks): plan_fp8_decode.  With k_new / v_new
// (float16 [B][H][d]) set, the launch also codes token T - 1 from them before reading it.
hipError_t launch_mx_decode(const MxView& L, int q_heads, int64_t T, const __half* q,
                            float sm_scale, float* out, void* ws, const Fp8Plan& plan,
                            const __half* k_new, const __half* v_new, hipStream_t s);

}  // namespace kivi
