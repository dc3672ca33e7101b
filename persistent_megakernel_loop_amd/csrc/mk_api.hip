// Host side of the C ABI declared in include/mk.h: validation, the weight arena,
// the KV cache, exchange buffers, the rotary table and the launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "mk.h"
#include "mk_internal.h"
#include "mk_prefill.h"

static_assert(MK_ID_RING == mk::kIdRing, "id ring size in mk.h");

using mk::LayerLayout;
using mk::Params;

// Poll rounds before a cross-workgroup wait gives up (about a second at the round times
// measured on MI355X).
constexpr uint32_t kDefaultSpinLimit = 1u << 22;

struct mk_handle {
  int body = -1;
  mk_cfg cfg{};
  hipStream_t stream = nullptr;
  int device = 0;
  int wb = 2;  // bytes per weight
  int kvb = 2; // bytes per cache entry
  // arena
  uint8_t* arena = nullptr;
  size_t arena_bytes = 0;
  LayerLayout lay{};
  uint8_t* embed = nullptr;
  uint8_t* lm_head = nullptr;
  float* in_norm0 = nullptr;
  float* rope_cos = nullptr;
  float* rope_sin = nullptr;
  // cache and exchange
  void* kcache = nullptr;
  void* vcache = nullptr;
  unsigned long long* xbuf = nullptr;
  size_t xbuf_words = 0;
  unsigned long long *xq, *xatt, *xop, *xxa, *xm, *xdp, *xxb, *xarg, *xplace, *xsink;
  uint32_t* ctl = nullptr;  // [0] err, [1] abort, [2] last id
  // pinned
  unsigned long long* progress = nullptr;
  unsigned long long* pinned_ids = nullptr;  // id ring [mk::kIdRing], entries mk::ring_entry
  // state
  int32_t pos = 0;
  bool have_last = false;
  uint32_t tag = 1;
  uint32_t lm_seq = 1;
  uint32_t call_seq = 0;
  float* dbg_hidden = nullptr;
  unsigned long long* dbg_trace = nullptr;
  unsigned long long* dbg_phase = nullptr;
  int32_t dbg_phase_wg = 0;
  uint32_t spin_limit = kDefaultSpinLimit;
  // batched prefill scratch, allocated by the first mk_prefill_batched call
  uint8_t* pf_buf = nullptr;
  uint32_t pf_tag = 1;   // next flag tag of the persistent prefill on pf_buf
  int32_t pf_path = 0;   // MK_PREFILL_AUTO / _CHAIN / _PERSISTENT
};

namespace {

struct BodyShape { int body, H, D, NQ, NKV, I, wdt; };
const BodyShape kBodies[] = {
    {mk::BODY_TINY, 256, 64, 4, 2, 768, MK_F32},
    {mk::BODY_Q06, 1024, 128, 16, 8, 3072, MK_BF16},
    {mk::BODY_Q17, 2048, 128, 16, 8, 6144, MK_BF16},
};

#define HIPCK(x)                          \
  do {                                    \
    if ((x) != hipSuccess) return MK_ERR_HIP; \
  } while (0)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int validate_cfg(const mk_cfg* c) {
  if (!c) return MK_ERR_ARG;
  if (c->n_layers <= 0 || c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->intermediate <= 0 || c->vocab <= 0 || c->max_seq <= 0)
    return MK_ERR_ARG;
  if (c->n_q_heads % c->n_kv_heads) return MK_ERR_ARG;
  if (c->head_dim % 2) return MK_ERR_ARG;
  if (c->weight_dtype != MK_F32 && c->weight_dtype != MK_BF16) return MK_ERR_ARG;
  if (c->kv_dtype != MK_F32 && c->kv_dtype != MK_BF16) return MK_ERR_ARG;
  if (c->n_sections < 1 || c->n_sections > 3) return MK_ERR_ARG;
  int sum = 0;
  for (int k = 0; k < c->n_sections; ++k) {
    if (c->sections[k] <= 0) return MK_ERR_ARG;
    sum += c->sections[k];
  }
  if (sum != c->head_dim / 2) return MK_ERR_ARG;
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return MK_ERR_ARG;
  if (c->vocab >= (1 << 18)) return MK_ERR_UNSUPPORTED;
  if (c->max_seq >= (1 << 26)) return MK_ERR_ARG;  // id ring entries hold slots below 2^26
  if ((long long)c->max_seq * c->n_layers * c->n_kv_heads * c->head_dim > (1ll << 40)) return MK_ERR_ARG;
  return MK_OK;
}

int pick_body(const mk_cfg* c) {
  for (const auto& b : kBodies)
    if (b.H == c->hidden && b.D == c->head_dim && b.NQ == c->n_q_heads && b.NKV == c->n_kv_heads &&
        b.I == c->intermediate && b.wdt == c->weight_dtype)
      return b.body;
  return -1;
}

// Layer layout of the packed arena (see the kernel's tile addressing).
LayerLayout make_layout(const mk_cfg* c, int wb) {
  const size_t H = c->hidden, D = c->head_dim, I = c->intermediate;
  const size_t NG = c->n_kv_heads, QPG = c->n_q_heads / c->n_kv_heads;
  const size_t RQKV = (QPG + 2) * D, OC = QPG * D, IX = I / mk::kXcds;
  LayerLayout L{};
  L.qkv = 0;
  L.o = align_up(L.qkv + NG * RQKV * H * wb, 256);
  L.gu = align_up(L.o + NG * H * OC * wb, 256);
  L.down = align_up(L.gu + mk::kXcds * 2 * IX * H * wb, 256);
  L.gains = align_up(L.down + mk::kXcds * H * IX * wb, 256);
  L.stride = align_up(L.gains + (2 * H + 2 * D) * 4, 4096);
  return L;
}

int copy2d(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height, hipStream_t s) {
  return hipMemcpy2DAsync(dst, dpitch, src, spitch, width, height, hipMemcpyDeviceToDevice, s) == hipSuccess ? MK_OK
                                                                                                            : MK_ERR_HIP;
}

// Pack one layer's weights into the arena tiles the kernel reads.
int pack_layer(mk_handle* h, const mk_weights* w, int l) {
  const mk_cfg* c = &h->cfg;
  const size_t H = c->hidden, D = c->head_dim, I = c->intermediate, wb = h->wb;
  const size_t NG = c->n_kv_heads, QPG = c->n_q_heads / c->n_kv_heads;
  const size_t RQKV = (QPG + 2) * D, OC = QPG * D, IX = I / mk::kXcds;
  const size_t HALF = IX / mk::kPerXcd;
  uint8_t* base = h->arena + (size_t)l * h->lay.stride;
  hipStream_t s = h->stream;
  const uint8_t* wq = (const uint8_t*)w->wq[l];
  const uint8_t* wk = (const uint8_t*)w->wk[l];
  const uint8_t* wv = (const uint8_t*)w->wv[l];
  const uint8_t* wo = (const uint8_t*)w->wo[l];
  const uint8_t* wg = (const uint8_t*)w->w_gate[l];
  const uint8_t* wu = (const uint8_t*)w->w_up[l];
  const uint8_t* wd = (const uint8_t*)w->w_down[l];
  const size_t row = H * wb;
  for (size_t g = 0; g < NG; ++g) {
    uint8_t* q = base + h->lay.qkv + g * RQKV * row;
    HIPCK(hipMemcpyAsync(q, wq + g * QPG * D * row, QPG * D * row, hipMemcpyDeviceToDevice, s));
    HIPCK(hipMemcpyAsync(q + QPG * D * row, wk + g * D * row, D * row, hipMemcpyDeviceToDevice, s));
    HIPCK(hipMemcpyAsync(q + (QPG + 1) * D * row, wv + g * D * row, D * row, hipMemcpyDeviceToDevice, s));
    // O columns of the group's heads: [H][OC]
    int e = copy2d(base + h->lay.o + g * H * OC * wb, OC * wb, wo + g * OC * wb, (size_t)c->n_q_heads * D * wb,
                   OC * wb, H, s);
    if (e) return e;
  }
  for (size_t x = 0; x < (size_t)mk::kXcds; ++x) {
    // workgroup r of XCD x: [HALF gate rows][HALF up rows], rows x*IX + r*HALF ...
    uint8_t* gu = base + h->lay.gu + x * 2 * IX * row;
    int e = copy2d(gu, 2 * HALF * row, wg + x * IX * row, HALF * row, HALF * row, mk::kPerXcd, s);
    if (e) return e;
    e = copy2d(gu + HALF * row, 2 * HALF * row, wu + x * IX * row, HALF * row, HALF * row, mk::kPerXcd, s);
    if (e) return e;
    // down columns of the slice: [H][IX]
    e = copy2d(base + h->lay.down + x * H * IX * wb, IX * wb, wd + x * IX * wb, I * wb, IX * wb, H, s);
    if (e) return e;
  }
  // gains block of layer l, in the order the kernel consumes it: post-attention norm, q norm,
  // k norm, then the input norm of layer l+1 (the final norm after the last layer)
  const int bf = c->weight_dtype == MK_BF16;
  float* g = (float*)(base + h->lay.gains);
  const void* next_in = l + 1 < c->n_layers ? w->in_norm[l + 1] : w->final_norm;
  if (mk::launch_widen(w->post_norm[l], g, (int)H, bf, s)) return MK_ERR_HIP;
  if (mk::launch_widen(w->q_norm[l], g + H, (int)D, bf, s)) return MK_ERR_HIP;
  if (mk::launch_widen(w->k_norm[l], g + H + D, (int)D, bf, s)) return MK_ERR_HIP;
  if (mk::launch_widen(next_in, g + H + 2 * D, (int)H, bf, s)) return MK_ERR_HIP;
  return MK_OK;
}

void free_handle(mk_handle* h) {
  if (!h) return;
  hipStreamSynchronize(h->stream);
  hipFree(h->arena);
  hipFree(h->kcache);
  hipFree(h->vcache);
  hipFree(h->xbuf);
  hipFree(h->ctl);
  hipFree(h->pf_buf);
  if (h->progress) hipHostFree(h->progress);
  if (h->pinned_ids) hipHostFree(h->pinned_ids);
  delete h;
}

int device_status(mk_handle* h, bool clear) {
  uint32_t ctl[2];
  HIPCK(hipStreamSynchronize(h->stream));
  HIPCK(hipMemcpy(ctl, h->ctl, sizeof ctl, hipMemcpyDeviceToHost));
  if (clear && (ctl[0] || ctl[1])) {
    uint32_t z[2] = {0, 0};
    HIPCK(hipMemcpy(h->ctl, z, sizeof z, hipMemcpyHostToDevice));
  }
  if (ctl[0] & mk::DEV_ERR_TIMEOUT) return MK_ERR_TIMEOUT;
  if (ctl[0]) return MK_ERR_DEVICE;
  if (ctl[1]) return MK_ERR_TIMEOUT;
  return MK_OK;
}

int run(mk_handle* h, int32_t n, const int32_t* ids, const float* rows, const int32_t* pos3, int32_t* out,
        int logits_from, int feedback, bool prompt, bool phased = false) {
  if (n <= 0) return MK_ERR_ARG;
  if ((long long)h->pos + n > h->cfg.max_seq) return MK_ERR_CAPACITY;
  if (feedback && !h->have_last) return MK_ERR_STATE;
  Params P{};
  P.layers = h->arena;
  P.lay = h->lay;
  P.embed = h->embed;
  P.lm_head = h->lm_head;
  P.in_norm0 = h->in_norm0;
  P.rope_cos = h->rope_cos;
  P.rope_sin = h->rope_sin;
  P.rope_positions = h->cfg.max_seq;
  P.n_layers = h->cfg.n_layers;
  P.vocab = h->cfg.vocab;
  P.max_seq = h->cfg.max_seq;
  P.n_sections = h->cfg.n_sections;
  P.sec_end0 = h->cfg.sections[0];
  P.sec_end1 = h->cfg.n_sections > 1 ? h->cfg.sections[0] + h->cfg.sections[1] : h->cfg.head_dim;
  if (h->cfg.n_sections == 1) P.sec_end0 = h->cfg.head_dim;  // every pair reads stream 0
  P.rms_eps = h->cfg.rms_eps;
  P.kcache = h->kcache;
  P.vcache = h->vcache;
  P.kv_bf16 = h->cfg.kv_dtype == MK_BF16;
  P.xq = h->xq; P.xatt = h->xatt; P.xop = h->xop; P.xxa = h->xxa;
  P.xm = h->xm; P.xdp = h->xdp; P.xxb = h->xxb; P.xarg = h->xarg;
  P.xplace = h->xplace;
  P.xsink = h->xsink;
  P.err = h->ctl;
  P.abort_flag = h->ctl + 1;
  P.last_id = (int32_t*)(h->ctl + 2);
  P.n_pos = n;
  P.pos0 = h->pos;
  P.logits_from = logits_from;
  P.feedback = feedback;
  P.ids = ids;
  P.rows = rows;
  P.pos3 = pos3;
  P.out_ids = out;
  P.pinned_ids = h->pinned_ids;
  h->call_seq += 1;
  P.call_seq = h->call_seq;
  P.progress = h->progress;
  P.dbg_hidden = h->dbg_hidden;
  P.dbg_trace = h->dbg_trace;
  P.dbg_phase = h->dbg_phase;
  P.dbg_phase_wg = h->dbg_phase_wg;
  // tags are compared for equality: before they wrap, clear the buffers so that no old word can match
  const uint32_t need = (uint32_t)n * mk::tags_per_position(h->cfg.n_layers) + 1;
  if ((unsigned long long)h->tag + need >= 0xFFFFFFF0ull) {
    if (hipMemsetAsync(h->xbuf, 0, h->xbuf_words * 8, h->stream) != hipSuccess) return MK_ERR_HIP;
    h->tag = 1;
  }
  P.tag0 = h->tag;
  P.lm_seq0 = h->lm_seq;
  P.spin_limit = h->spin_limit;
  P.whole = mk::whole_call(h->body, h->pos, n) ? 1 : 0;
  if (phased) {
    const int e = mk::launch_phased(h->body, P, h->stream);
    if (e == -2) return MK_ERR_UNSUPPORTED;
    if (e) return MK_ERR_HIP;
  } else if (mk::launch_decode(h->body, P, prompt, h->stream)) {
    return MK_ERR_HIP;
  }
  h->tag += need;
  h->lm_seq = (h->lm_seq + (uint32_t)(n - logits_from)) & 0x3fffu;
  h->pos += n;
  h->have_last = true;
  return MK_OK;
}


// Byte offsets of the batched prefill's scratch regions (activations, their bf16 split,
// queries, sums of squares, LM-head block maxima, attention and product partials) for a
// handle's shape; `bytes` is the whole.  0 bytes: the shape is not supported.
// The persistent form's regions (pp[1..9], after its flag words pp[0]) overlay the
// chain's (xs .. part): a chunk runs one form or the other.  The flag words come first
// and nothing else is ever written there, and x, which the LM head reads after either
// form, lies outside the overlay.
struct PfScratch { size_t flags, x, blk_val, blk_idx, xs, q, ss, att, part, pp[10], bytes; bool pp_ok; };

PfScratch pf_scratch(const mk_cfg* c) {
  PfScratch r{};
  const size_t part = mk::prefill_part_floats(c->hidden, c->n_q_heads, c->n_kv_heads, c->head_dim, c->intermediate);
  if (c->weight_dtype != MK_BF16 || c->head_dim != 128 || c->n_q_heads != 2 * c->n_kv_heads || part == 0 ||
      c->hidden % 512 || c->hidden > 2048 || c->intermediate % 1024)
    return r;
  const size_t ch = mk::kPrefillChunk, H = c->hidden;
  const size_t K = std::max<size_t>(std::max<size_t>(H, (size_t)c->n_q_heads * c->head_dim), (size_t)c->intermediate);
  const size_t n_blk = (size_t)(c->vocab + mk::kLmRowsPerBlock - 1) / mk::kLmRowsPerBlock;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += align_up(bytes, 256); return at; };
  size_t pp[10];
  const size_t pp_total = mk::pp_layout(c->hidden, c->n_q_heads, c->n_kv_heads, c->head_dim, c->intermediate, pp);
  r.pp_ok = pp_total > 0;
  r.flags = take((size_t)mk::kPpKinds * mk::kGrid * 8);
  r.x = take(ch * H * 4);
  r.blk_val = take(n_blk * 4);
  r.blk_idx = take(n_blk * 4);
  const size_t overlay = off;
  r.xs = take(2 * K * ch * 2);
  r.q = take(ch * c->n_q_heads * c->head_dim * 4);
  r.ss = take(ch * (H / 512) * 4);
  r.att = take((size_t)c->n_kv_heads * mk::kFlashRanges * 2 * ch * (c->head_dim + 2) * 4);
  r.part = take(part * 4);
  if (r.pp_ok) {
    r.pp[0] = r.flags;
    for (int k = 1; k < 10; ++k) r.pp[k] = overlay + (pp[k] - pp[1]);
    off = std::max(off, overlay + align_up(pp_total - pp[1], 256));
  }
  r.bytes = off;
  return r;
}

// Every batched prefill step on scratch `buf` (pf_scratch(&h->cfg).bytes bytes of device
// memory).  Each scratch word the launches read was written earlier in the same call, so
// the buffer needs no clearing.  Allocates nothing.
// Which form runs a call: the persistent one where the handle allows it and every chunk
// qualifies (the shape has the form, and the context ends at or below kPpMaxKeys), else
// the kernel chain.  -1: the handle asks for the persistent form and the call has none.
int prefill_form(const mk_handle* h, const PfScratch& S, int32_t n) {
  const bool fits = S.pp_ok && (long long)h->pos + n <= mk::kPpMaxKeys;
  if (h->pf_path == MK_PREFILL_CHAIN) return 0;
  if (h->pf_path == MK_PREFILL_PERSISTENT) return fits ? 1 : -1;
  return fits ? 1 : 0;
}

int prefill_batched(mk_handle* h, uint8_t* buf, const PfScratch& S, const int32_t* d_ids, const float* d_rows,
                    const int32_t* d_pos3, int32_t n, int32_t* d_out_first, uint32_t* tag) {
  const mk_cfg* c = &h->cfg;
  const int form = prefill_form(h, S, n);
  if (form < 0) return MK_ERR_UNSUPPORTED;
  mk::PpBufs B{};
  if (form == 1) {
    B.flags = (unsigned long long*)(buf + S.pp[0]);
    B.xb = (uint16_t*)(buf + S.pp[1]);
    B.xp = (uint16_t*)(buf + S.pp[2]);
    B.ss = (float*)(buf + S.pp[3]);
    B.ss2 = (float*)(buf + S.pp[4]);
    B.qr = (float*)(buf + S.pp[5]);
    B.at = (uint16_t*)(buf + S.pp[6]);
    B.op = (float*)(buf + S.pp[7]);
    B.hs = (uint16_t*)(buf + S.pp[8]);
    B.dp = (float*)(buf + S.pp[9]);
  }
  const int ch = mk::kPrefillChunk;
  const size_t H = c->hidden;
  mk::PfArgs A{};
  A.H = c->hidden; A.D = c->head_dim; A.NQ = c->n_q_heads; A.NKV = c->n_kv_heads; A.I = c->intermediate;
  A.L = c->n_layers; A.vocab = c->vocab; A.max_seq = c->max_seq; A.rope_positions = c->max_seq;
  A.n_sections = c->n_sections;
  A.sec_end0 = c->n_sections == 1 ? c->head_dim : c->sections[0];
  A.sec_end1 = c->n_sections > 1 ? c->sections[0] + c->sections[1] : c->head_dim;
  A.eps = c->rms_eps;
  A.embed = (const uint16_t*)h->embed;
  A.in_norm0 = h->in_norm0;
  A.rope_cos = h->rope_cos;
  A.rope_sin = h->rope_sin;
  A.kcache = (uint16_t*)h->kcache;  // bf16: mk_create ties the cache dtype to the weight dtype
  A.vcache = (uint16_t*)h->vcache;
  A.err = h->ctl;
  A.x = (float*)(buf + S.x);
  A.xs = (uint16_t*)(buf + S.xs);
  A.part = (float*)(buf + S.part);
  A.q = (float*)(buf + S.q);
  A.ss = (float*)(buf + S.ss);
  A.att = (float*)(buf + S.att);
  for (int32_t t0 = 0; t0 < n; t0 += ch) {
    A.m = std::min(ch, n - t0);
    A.npp = (A.m + 15) / 16 * 16;
    A.pos0 = h->pos + t0;
    A.ids = d_ids + t0;
    A.rows = d_rows ? d_rows + (size_t)t0 * H : nullptr;
    A.pos3 = d_pos3 ? d_pos3 + (size_t)t0 * 3 : nullptr;
    A.dbg_hidden = h->dbg_hidden ? h->dbg_hidden + (size_t)t0 * (c->n_layers + 1) * H : nullptr;
    if (form == 1) {
      // flag tags of this launch: (L + 1) * kPpKinds, all above every tag the words hold;
      // past the top of the range the words are cleared (stream-ordered) and tags restart
      const uint32_t need = (uint32_t)(c->n_layers + 1) * mk::kPpKinds;
      if ((unsigned long long)*tag + need >= 0xFFFFFF00ull) {
        if (mk::launch_pp_clear(B.flags, h->stream)) return MK_ERR_HIP;
        *tag = 1;
      }
      if (mk::launch_prefill_persistent(A, B, h->arena, h->lay, *tag, h->spin_limit, h->ctl + 1, h->dbg_phase,
                                        h->stream))
        return MK_ERR_HIP;
      *tag += need;
    } else if (mk::launch_prefill_chunk(A, h->arena, h->lay, h->stream)) {
      return MK_ERR_HIP;
    }
  }
  // the last chunk's residual stream is still in place: its last row gives the first id
  const uint8_t* last_layer = h->arena + (size_t)(c->n_layers - 1) * h->lay.stride;
  mk::LmArgs M{};
  M.lm_head = (const uint16_t*)h->lm_head;
  M.g_final = (const float*)(last_layer + h->lay.gains) + H + 2 * c->head_dim;
  M.n_last = A.m - 1;
  M.blk_val = (float*)(buf + S.blk_val);
  M.blk_idx = (int32_t*)(buf + S.blk_idx);
  M.out_first = d_out_first;
  M.last_id = (int32_t*)(h->ctl + 2);
  M.pinned_ids = h->pinned_ids;
  M.progress = h->progress;
  h->call_seq += 1;
  M.call_seq = h->call_seq;
  if (mk::launch_prefill_lm(A, M, h->stream)) return MK_ERR_HIP;
  h->pos += n;
  h->have_last = true;
  return MK_OK;
}

// Scratch of mk_prefill_batched_noalloc: a fixed array that every device the library
// runs on holds from the code object's load until the process ends.  Host code never
// passes its name to a kernel: the name is a host-side stand-in, and the device address
// comes from scratch_setup.
constexpr size_t kStaticScratchBytes = (size_t)MK_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device; NULL before set-up
uint32_t g_scratch_tag[kMaxDevices];  // next flag tag of the persistent prefill on each device's `scratch`

// Looks up the address of `scratch` on `dev`, which must be the current device; once
// per device.
int scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return MK_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return MK_OK;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
    (void)hipGetLastError();
    return MK_ERR_HIP;
  }
  g_scratch_ptr[dev] = (uint8_t*)ptr;
  g_scratch_tag[dev] = 1;  // the array starts zeroed, like every device variable without initializer
  return MK_OK;
}

uint8_t* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[dev];
}

int prefill_batched_args(mk_handle* h, const int32_t* d_ids, int32_t n, int32_t* d_out_first, PfScratch* S) {
  if (!h || !d_ids || n <= 0 || !d_out_first) return MK_ERR_ARG;
  if ((long long)h->pos + n > h->cfg.max_seq) return MK_ERR_CAPACITY;
  *S = pf_scratch(&h->cfg);
  if (S->bytes == 0) return MK_ERR_UNSUPPORTED;
  return MK_OK;
}

}  // namespace

extern "C" {

int mk_create(const mk_weights* w, const mk_cfg* cfg, void* stream, mk_handle** out) {
  if (!out) return MK_ERR_ARG;
  *out = nullptr;
  if (!w) return MK_ERR_ARG;
  int e = validate_cfg(cfg);
  if (e) return e;
  const int L = cfg->n_layers;
  if (!w->embed || !w->final_norm || (!cfg->tied && !w->lm_head)) return MK_ERR_ARG;
  const void* const* arrs[] = {w->in_norm, w->wq, w->wk, w->wv, w->q_norm, w->k_norm, w->wo, w->post_norm,
                               w->w_gate, w->w_up, w->w_down};
  for (auto a : arrs) {
    if (!a) return MK_ERR_ARG;
    for (int l = 0; l < L; ++l)
      if (!a[l]) return MK_ERR_ARG;
  }
  const int body = pick_body(cfg);
  if (body < 0) return MK_ERR_UNSUPPORTED;
  if (cfg->kv_dtype != cfg->weight_dtype) return MK_ERR_UNSUPPORTED;  // each body caches in its weight dtype
  int blocks = 0;
  if (mk::coop_ok(body, &blocks)) return MK_ERR_HIP;
  mk_handle* h = new (std::nothrow) mk_handle();
  if (!h) return MK_ERR_OOM;
  h->body = body;
  h->cfg = *cfg;
  h->stream = (hipStream_t)stream;
  h->wb = cfg->weight_dtype == MK_BF16 ? 2 : 4;
  h->kvb = cfg->kv_dtype == MK_BF16 ? 2 : 4;
  hipGetDevice(&h->device);
  if (scratch_setup(h->device)) { free_handle(h); return MK_ERR_HIP; }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, h->device) != hipSuccess) { free_handle(h); return MK_ERR_HIP; }
  if (prop.multiProcessorCount != mk::kGrid || blocks < 1 || !prop.cooperativeLaunch) { free_handle(h); return MK_ERR_COOP; }

  const size_t H = cfg->hidden, D = cfg->head_dim, V = cfg->vocab;
  h->lay = make_layout(cfg, h->wb);
  size_t off = (size_t)L * h->lay.stride;
  const size_t embed_off = off;
  off = align_up(off + V * H * h->wb, 4096);
  size_t lm_off = embed_off;
  if (!cfg->tied) { lm_off = off; off = align_up(off + V * H * h->wb, 4096); }
  const size_t fn_off = off;
  off = align_up(off + H * 4, 256);
  const size_t rope_off = off;
  const size_t rope_n = (size_t)cfg->max_seq * (D / 2);
  off = align_up(off + 2 * rope_n * 4, 256);
  h->arena_bytes = off;
  if (hipMalloc((void**)&h->arena, h->arena_bytes) != hipSuccess) { free_handle(h); return MK_ERR_OOM; }
  h->embed = h->arena + embed_off;
  h->lm_head = h->arena + lm_off;
  h->in_norm0 = (float*)(h->arena + fn_off);
  h->rope_cos = (float*)(h->arena + rope_off);
  h->rope_sin = h->rope_cos + rope_n;

  const size_t kv_bytes = (size_t)L * cfg->n_kv_heads * cfg->max_seq * D * h->kvb;
  if (hipMalloc(&h->kcache, kv_bytes) != hipSuccess || hipMalloc(&h->vcache, kv_bytes) != hipSuccess) {
    free_handle(h);
    return MK_ERR_OOM;
  }
  // exchange buffers
  const size_t QPG = cfg->n_q_heads / cfg->n_kv_heads, IX = cfg->intermediate / mk::kXcds;
  const size_t nq = 8 * (QPG + 2) * D, natt = 8 * mk::kPerXcd * QPG * (D + 2), nh = 8 * H, nm = 8 * IX;
  h->xbuf_words = nq + natt + 5 * nh + nm + 2 * mk::kGrid + 64 * mk::kGrid + 64 * 10;
  if (hipMalloc((void**)&h->xbuf, h->xbuf_words * 8) != hipSuccess ||
      hipMalloc((void**)&h->ctl, 256) != hipSuccess) {
    free_handle(h);
    return MK_ERR_OOM;
  }
  unsigned long long* p = h->xbuf;
  auto take = [&](size_t n) { unsigned long long* r = p; p += align_up(n, 64); return r; };
  h->xq = take(nq); h->xatt = take(natt); h->xop = take(nh); h->xxa = take(nh); h->xm = take(nm);
  h->xdp = take(nh); h->xxb = take(nh); h->xarg = take(mk::kGrid);
  h->xplace = take(mk::kGrid);
  h->xsink = take(64 * mk::kGrid);
  if ((size_t)(p - h->xbuf) > h->xbuf_words) { free_handle(h); return MK_ERR_ARG; }
  if (hipHostMalloc((void**)&h->progress, 64, hipHostMallocCoherent) != hipSuccess) { free_handle(h); return MK_ERR_OOM; }
  *(volatile unsigned long long*)h->progress = 0;
  if (hipHostMalloc((void**)&h->pinned_ids, sizeof(unsigned long long) * mk::kIdRing, hipHostMallocCoherent) !=
      hipSuccess) {
    h->pinned_ids = nullptr;
    free_handle(h);
    return MK_ERR_OOM;
  }
  std::memset(h->pinned_ids, 0, sizeof(unsigned long long) * mk::kIdRing);

  hipStream_t s = h->stream;
  if (hipMemsetAsync(h->xbuf, 0, h->xbuf_words * 8, s) != hipSuccess || hipMemsetAsync(h->ctl, 0, 256, s) != hipSuccess) {
    free_handle(h);
    return MK_ERR_HIP;
  }
  for (int l = 0; l < L; ++l) {
    e = pack_layer(h, w, l);
    if (e) { free_handle(h); return e; }
  }
  if (hipMemcpyAsync(h->embed, w->embed, V * H * h->wb, hipMemcpyDeviceToDevice, s) != hipSuccess ||
      (!cfg->tied && hipMemcpyAsync(h->lm_head, w->lm_head, V * H * h->wb, hipMemcpyDeviceToDevice, s) != hipSuccess) ||
      mk::launch_widen(w->in_norm[0], h->in_norm0, (int)H, cfg->weight_dtype == MK_BF16, s)) {
    free_handle(h);
    return MK_ERR_HIP;
  }
  // rotary table: cos/sin of pos * theta^(-2i/d), computed in double, stored as float
  std::vector<float> tab(2 * rope_n);
  for (size_t ps = 0; ps < (size_t)cfg->max_seq; ++ps)
    for (size_t i = 0; i < D / 2; ++i) {
      const double ang = (double)ps * std::pow((double)cfg->rope_theta, -2.0 * (double)i / (double)D);
      tab[ps * (D / 2) + i] = (float)std::cos(ang);
      tab[rope_n + ps * (D / 2) + i] = (float)std::sin(ang);
    }
  if (hipMemcpyAsync(h->rope_cos, tab.data(), tab.size() * 4, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    free_handle(h);
    return MK_ERR_HIP;
  }
  *out = h;
  return MK_OK;
}

int mk_prefill(mk_handle* h, const int32_t* d_ids, const float* d_rows, const int32_t* d_pos3, int32_t n,
               int32_t* d_out_first) {
  if (!h || !d_ids || n <= 0) return MK_ERR_ARG;
  return run(h, n, d_ids, d_rows, d_pos3, d_out_first, n - 1, 0, true);
}

int mk_prefill_batched(mk_handle* h, const int32_t* d_ids, const float* d_rows, const int32_t* d_pos3, int32_t n,
                       int32_t* d_out_first) {
  PfScratch S;
  int e = prefill_batched_args(h, d_ids, n, d_out_first, &S);
  if (e) return e;
  if (!h->pf_buf) {
    if (hipMalloc((void**)&h->pf_buf, S.bytes) != hipSuccess) {
      h->pf_buf = nullptr;
      return MK_ERR_OOM;
    }
    // the persistent form's flag words start at zero, below every tag
    if (mk::launch_pp_clear((unsigned long long*)(h->pf_buf + S.flags), h->stream)) return MK_ERR_HIP;
    h->pf_tag = 1;
  }
  return prefill_batched(h, h->pf_buf, S, d_ids, d_rows, d_pos3, n, d_out_first, &h->pf_tag);
}

int mk_prefill_batched_noalloc(mk_handle* h, const int32_t* d_ids, const float* d_rows, const int32_t* d_pos3,
                               int32_t n, int32_t* d_out_first) {
  PfScratch S;
  int e = prefill_batched_args(h, d_ids, n, d_out_first, &S);
  if (e) return e;
  if (S.bytes > kStaticScratchBytes) return MK_ERR_SCRATCH;
  uint8_t* buf = scratch_ptr(h->device);
  if (!buf) return MK_ERR_STATE;  // mk_create looks the address up on the handle's device
  std::lock_guard<std::mutex> lock(g_scratch_mu);  // the device's tag counter
  return prefill_batched(h, buf, S, d_ids, d_rows, d_pos3, n, d_out_first, &g_scratch_tag[h->device]);
}

int mk_decode(mk_handle* h, int32_t n_steps, const int32_t* d_ids, const float* d_embed_buf, const int32_t* d_pos3,
              int32_t* d_out_ids) {
  if (!h || n_steps <= 0 || !d_out_ids) return MK_ERR_ARG;
  return run(h, n_steps, d_ids, d_embed_buf, d_pos3, d_out_ids, 0, d_ids == nullptr, false);
}

int mk_decode_phased(mk_handle* h, int32_t n_steps, const int32_t* d_ids, const float* d_embed_buf,
                     const int32_t* d_pos3, int32_t* d_out_ids) {
  if (!h || n_steps <= 0 || !d_out_ids) return MK_ERR_ARG;
  if (h->body != mk::BODY_Q06) return MK_ERR_UNSUPPORTED;
  return run(h, n_steps, d_ids, d_embed_buf, d_pos3, d_out_ids, 0, d_ids == nullptr, false, true);
}

int mk_load_kv(mk_handle* h, const void* d_kv, int32_t n_pos) {
  if (!h || !d_kv || n_pos < 0) return MK_ERR_ARG;
  if (n_pos > h->cfg.max_seq) return MK_ERR_CAPACITY;
  const size_t D = h->cfg.head_dim, NKV = h->cfg.n_kv_heads, row = D * h->kvb;
  const uint8_t* src = (const uint8_t*)d_kv;
  for (int l = 0; l < h->cfg.n_layers; ++l)
    for (int kv = 0; kv < 2; ++kv) {
      // source [l][kv][g][n_pos][D] -> cache [l][g][max_seq][D]; one 2D copy per (l, kv)
      uint8_t* dst = (uint8_t*)(kv ? h->vcache : h->kcache) + (size_t)l * NKV * h->cfg.max_seq * row;
      const uint8_t* s0 = src + (((size_t)l * 2 + kv) * NKV) * n_pos * row;
      if (n_pos && copy2d(dst, (size_t)h->cfg.max_seq * row, s0, (size_t)n_pos * row, (size_t)n_pos * row, NKV,
                          h->stream))
        return MK_ERR_HIP;
    }
  h->pos = n_pos;
  h->have_last = false;
  return MK_OK;
}

int mk_reset(mk_handle* h) {
  if (!h) return MK_ERR_ARG;
  // re-arm the device side too (stream-ordered): the error word, the abort flag a timed-out
  // wait raised (every later wait would give up early otherwise) and the timeout record
  if (hipMemsetAsync(h->ctl, 0, 2 * sizeof(uint32_t), h->stream) != hipSuccess ||
      hipMemsetAsync(h->ctl + 3, 0, 5 * sizeof(uint32_t), h->stream) != hipSuccess)
    return MK_ERR_HIP;
  h->pos = 0;
  h->have_last = false;
  return MK_OK;
}

int mk_position(mk_handle* h, int32_t* pos) {
  if (!h || !pos) return MK_ERR_ARG;
  *pos = h->pos;
  return MK_OK;
}

int mk_set_debug(mk_handle* h, float* d_hidden, uint64_t* d_trace) {
  if (!h) return MK_ERR_ARG;
  h->dbg_hidden = d_hidden;
  h->dbg_trace = (unsigned long long*)d_trace;
  return MK_OK;
}

int mk_set_prefill_path(mk_handle* h, int32_t path) {
  if (!h || path < MK_PREFILL_AUTO || path > MK_PREFILL_PERSISTENT) return MK_ERR_ARG;
  h->pf_path = path;
  return MK_OK;
}

int mk_set_spin_limit(mk_handle* h, uint32_t polls) {
  if (!h) return MK_ERR_ARG;
  h->spin_limit = polls ? polls : kDefaultSpinLimit;
  return MK_OK;
}

int mk_set_phase_trace(mk_handle* h, uint64_t* d_phase, int32_t wg) {
  if (!h || wg < -1 || wg >= mk::kGrid) return MK_ERR_ARG;
  h->dbg_phase = (unsigned long long*)d_phase;
  h->dbg_phase_wg = wg;
  return MK_OK;
}

int mk_progress(mk_handle* h, int64_t* steps_done) {
  if (!h || !steps_done) return MK_ERR_ARG;
  const unsigned long long v = *(volatile unsigned long long*)h->progress;
  *steps_done = (uint32_t)(v >> 32) == h->call_seq ? (int64_t)(v & 0xffffffffu) : 0;
  return MK_OK;
}

int mk_read_ids(mk_handle* h, int32_t first, int32_t count, int32_t* host_out) {
  if (!h || !host_out || first < 0 || count < 0) return MK_ERR_ARG;
  int64_t done = 0;
  mk_progress(h, &done);
  if ((int64_t)first + count > done) return MK_ERR_ARG;
  // every entry carries its call and lap: an entry still behind the progress word (the two
  // stores are not ordered on the device) is read again until it arrives; one of a later
  // lap means the ring has already moved past it
  std::atomic_thread_fence(std::memory_order_acquire);
  const volatile unsigned long long* m = h->pinned_ids;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t s = first + i;
    const unsigned long long want = mk::ring_entry(h->call_seq, s, 0) >> 18;  // call and lap
    for (int spin = 0;; ++spin) {
      const unsigned long long v = m[s & (mk::kIdRing - 1)];
      if ((v >> 18) == want) {
        host_out[i] = (int32_t)(v & 0x3ffff);
        break;
      }
      if ((v >> 32) == h->call_seq && (v >> 18) > want) return MK_ERR_OVERRUN;
      if (spin == 10000000) return MK_ERR_TIMEOUT;
    }
  }
  return MK_OK;
}

int mk_query(mk_handle* h, int32_t* idle) {
  if (!h || !idle) return MK_ERR_ARG;
  const hipError_t e = hipStreamQuery(h->stream);
  if (e == hipSuccess) { *idle = 1; return MK_OK; }
  if (e == hipErrorNotReady) { *idle = 0; return MK_OK; }
  return MK_ERR_HIP;
}

int mk_status(mk_handle* h) {
  if (!h) return MK_ERR_ARG;
  return device_status(h, true);
}

int mk_error_info(mk_handle* h, int32_t* info) {
  if (!h || !info) return MK_ERR_ARG;
  uint32_t c[8];
  HIPCK(hipStreamSynchronize(h->stream));
  HIPCK(hipMemcpy(c, h->ctl, sizeof c, hipMemcpyDeviceToHost));
  info[0] = (int32_t)c[3];
  for (int k = 1; k < 5; ++k) info[k] = (int32_t)c[3 + k];
  const uint32_t z = 0;
  HIPCK(hipMemcpy(h->ctl + 3, &z, sizeof z, hipMemcpyHostToDevice));  // re-arm the record
  return MK_OK;
}

int mk_selftest_lds_dma(const void* d_src, void* d_dst, int32_t n_chunks, int32_t offset_bytes, void* stream) {
  if (!d_src || !d_dst || n_chunks <= 0 || offset_bytes < 0 || offset_bytes % 16 ||
      offset_bytes + 16 * n_chunks > 144 * 1024)
    return MK_ERR_ARG;
  return mk::launch_lds_dma_selftest(d_src, d_dst, n_chunks, offset_bytes, stream) ? MK_ERR_HIP : MK_OK;
}

int mk_selftest_gemm(const void* d_w, int32_t rows, int32_t k, const float* d_x, int32_t n, float* d_y, void* stream) {
  if (!d_w || !d_x || !d_y || rows <= 0 || k <= 0 || rows % 32 || k % 64 || n <= 0 || n > mk::kPrefillChunk)
    return MK_ERR_ARG;
  const size_t npp = (size_t)(n + 15) / 16 * 16;
  uint8_t* buf = nullptr;
  const size_t bxs = align_up(2 * (size_t)k * npp * 2, 256), bp = (size_t)k / 64 * npp * rows * 4;
  if (hipMalloc((void**)&buf, bxs + bp) != hipSuccess) return MK_ERR_OOM;
  int e = mk::launch_gemm_selftest((const uint16_t*)d_w, rows, k, d_x, n, d_y, (uint16_t*)buf, (float*)(buf + bxs), stream)
              ? MK_ERR_HIP : MK_OK;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) e = MK_ERR_HIP;
  hipFree(buf);
  return e;
}

int mk_bench_stream_read(const void* d_src, uint64_t bytes, int32_t nontemporal, uint64_t* d_sink, int32_t blocks,
                         void* stream) {
  if (!d_src || !d_sink || bytes < 16 || bytes % 16 || blocks <= 0 || blocks > 65536) return MK_ERR_ARG;
  return mk::launch_stream_read(d_src, (size_t)bytes, nontemporal, (unsigned long long*)d_sink, blocks, stream)
             ? MK_ERR_HIP
             : MK_OK;
}

int mk_selftest_exchange(int32_t iters, uint32_t spin_limit, int32_t xcd_local, uint32_t* result, void* stream) {
  if (iters <= 0 || !result) return MK_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  const size_t n_words = 2 * (size_t)mk::kGrid * 64 + mk::kGrid;  // two rounds' words, then the placement words
  unsigned long long* words = nullptr;
  uint32_t* ctl = nullptr;
  if (hipMalloc((void**)&words, n_words * 8) != hipSuccess) return MK_ERR_OOM;
  if (hipMalloc((void**)&ctl, 256) != hipSuccess) {
    hipFree(words);
    return MK_ERR_OOM;
  }
  int e = MK_OK;
  if (hipMemsetAsync(words, 0, n_words * 8, st) != hipSuccess || hipMemsetAsync(ctl, 0, 256, st) != hipSuccess)
    e = MK_ERR_HIP;
  Params P{};
  P.tag0 = 1;
  P.spin_limit = spin_limit ? spin_limit : kDefaultSpinLimit;
  P.err = ctl;
  P.abort_flag = ctl + 1;
  P.xq = words;
  uint32_t* bad = ctl + 16;  // [0] mismatched words, [1] workgroups whose wait gave up, [2] plain stores used
  if (e == MK_OK && mk::launch_exchange_stress(P, words, words + 2 * (size_t)mk::kGrid * 64, iters, xcd_local != 0,
                                               bad, st))
    e = MK_ERR_COOP;
  uint32_t host[19] = {0};
  if (hipStreamSynchronize(st) != hipSuccess || hipMemcpy(host, ctl, sizeof host, hipMemcpyDeviceToHost) != hipSuccess)
    e = MK_ERR_HIP;
  result[0] = host[16];
  result[1] = host[17];
  result[2] = host[0];
  result[3] = host[18];
  hipFree(words);
  hipFree(ctl);
  return e;
}

int mk_grid_size(mk_handle* h, int32_t* n) {
  if (!h || !n) return MK_ERR_ARG;
  *n = mk::kGrid;
  return MK_OK;
}

int mk_embed_sum(const void* d_codebooks, int32_t n_codebooks, int32_t codebook_size, const void* d_text,
                 int32_t text_vocab, int32_t hidden, int32_t dtype, const int32_t* d_ids, int32_t n, float* d_rows,
                 int32_t* d_bad, void* stream) {
  if (n < 0 || n_codebooks <= 0 || codebook_size <= 0 || text_vocab <= 0 || hidden <= 0 ||
      (dtype != MK_F32 && dtype != MK_BF16))
    return MK_ERR_ARG;
  if (n == 0) return MK_OK;  // nothing to read or write: the pointers may be NULL
  if (!d_codebooks || !d_text || !d_ids || !d_rows) return MK_ERR_ARG;
  return mk::launch_embed_sum(d_codebooks, n_codebooks, codebook_size, d_text, text_vocab, hidden,
                              dtype == MK_BF16, d_ids, n, d_rows, d_bad, stream)
             ? MK_ERR_HIP
             : MK_OK;
}

const char* mk_strerror(int code) {
  switch (code) {
    case MK_OK: return "ok";
    case MK_ERR_ARG: return "invalid argument";
    case MK_ERR_UNSUPPORTED: return "configuration has no compiled kernel body";
    case MK_ERR_OOM: return "out of memory";
    case MK_ERR_CAPACITY: return "KV cache capacity exceeded";
    case MK_ERR_COOP: return "one workgroup per CU cannot be co-resident";
    case MK_ERR_HIP: return "HIP runtime error";
    case MK_ERR_DEVICE: return "device reported a bad id or position";
    case MK_ERR_TIMEOUT: return "device wait timed out";
    case MK_ERR_STATE: return "no previous id for feedback decode";
    case MK_ERR_SCRATCH: return "shape needs more scratch than the fixed array holds";
    case MK_ERR_OVERRUN: return "the id ring moved past ids not yet read";
  }
  return "unknown error";
}

void mk_destroy(mk_handle* h) { free_handle(h); }

}  // extern "C"
