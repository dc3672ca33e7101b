// Internal declarations shared by the host library and the persistent kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mk {

// Grid geometry: one workgroup per CU, 8 XCDs of 32 CUs on MI355X.  Workgroups are
// dispatched round-robin over the XCDs, so workgroup b runs on XCD b % 8 and is
// rank b / 8 inside it.  Correctness never depends on that placement (all
// cross-workgroup traffic is device-coherent); only locality does.
constexpr int kXcds = 8;
constexpr int kPerXcd = 32;
constexpr int kGrid = kXcds * kPerXcd;
constexpr int kWorkerWaves = 7;              // stream weights and do the dot products
constexpr int kThreads = (kWorkerWaves + 1) * 64;  // + one control wave (polls, exchanges): 8 waves,
                                                   // two per SIMD, so each wave may use 256 VGPRs

enum BodyId : int { BODY_TINY = 0, BODY_Q06 = 1, BODY_Q17 = 2 };

// Device error word values (bit flags).
enum : uint32_t { DEV_ERR_ID = 1u, DEV_ERR_POS = 2u, DEV_ERR_TIMEOUT = 4u };

// Offsets (bytes) of one layer's tensors inside the arena; every layer has the same layout.
struct LayerLayout {
  size_t qkv, o, gu, down;            // packed weight tiles (weight dtype)
  size_t gains;                        // float32 block [post H][q_norm D][k_norm D][next input norm H]
  size_t stride;                       // bytes per layer
};

struct Params {
  // weights
  const uint8_t* layers;     // arena base of layer 0
  LayerLayout lay;
  const void* embed;         // [V][H] weight dtype
  const void* lm_head;       // [V][H] weight dtype (== embed when tied)
  const float* in_norm0;     // [H] input norm of layer 0 (the next-input norm of layer L-1 is the final norm)
  const float* rope_cos;     // [rope_positions][D/2]
  const float* rope_sin;
  int32_t rope_positions;
  // shape (runtime part)
  int32_t n_layers, vocab, max_seq;
  int32_t n_sections, sec_end0, sec_end1;  // pair i < sec_end0 -> stream 0, < sec_end1 -> 1, else 2
  float rms_eps;
  // KV cache [L][NKV][max_seq][D] for K and for V, kv dtype
  void* kcache;
  void* vcache;
  int32_t kv_bf16;
  // exchange buffers (64-bit tagged words, zero-initialised)
  unsigned long long* xq;    // [8][QKV rows per XCD]          local hop
  unsigned long long* xatt;  // [8][32][QPG][D+2]               local hop
  unsigned long long* xop;   // [32][NG][H/32] O partials, by reader      cross hop
  unsigned long long* xxa;   // [8][H] residual after attention local hop
  unsigned long long* xm;    // [8][I/8]                         local hop
  unsigned long long* xdp;   // [32][8][H/32] down partials, by reader    cross hop
  unsigned long long* xxb;   // [8][H] residual after the MLP    local hop
  unsigned long long* xarg;  // [grid] argmax keys               cross hop
  unsigned long long* xplace;  // [grid] XCD of every workgroup, once per launch
  unsigned long long* xsink;   // [grid][64] never read: lanes with nothing to publish store here
  uint32_t* err;             // device error word; err[3..7]: where the first timeout happened
  uint32_t* abort_flag;      // set on timeout: every wait gives up
  int32_t* last_id;          // feedback id carried between launches
  // this launch
  int32_t n_pos;             // positions to run
  int32_t pos0;              // first position
  int32_t logits_from;       // run the LM head for t >= logits_from (decode: 0; prefill: n-1)
  int32_t feedback;          // 1: input id of step t>0 is the argmax of step t-1; step 0 reads *last_id
  const int32_t* ids;        // [n_pos] or NULL (feedback)
  const float* rows;         // [n_pos][H] or NULL
  const int32_t* pos3;       // [n_pos][3] or NULL
  int32_t* out_ids;          // [n_pos - logits_from] or NULL
  unsigned long long* pinned_ids;  // host-pinned id ring [kIdRing] (ring_entry), or NULL
  unsigned long long* progress;  // host-pinned step counter
  float* dbg_hidden;         // [n_pos][L+1][H] or NULL
  unsigned long long* dbg_trace; // [n_pos][grid][2] or NULL
  unsigned long long* dbg_phase; // barrier timeline: [n_pos][2 + 10 L][8] of one workgroup, or NULL
  int32_t dbg_phase_wg;          // the traced workgroup; -1: all, [n_pos][grid][2 + 10 L][8]
  uint32_t tag0;             // first exchange tag of this launch
  uint32_t lm_seq0;          // argmax key sequence of the first LM head of this launch (14 bits used)
  uint32_t call_seq;         // high half of the progress word
  uint32_t spin_limit;       // polls before a wait gives up
  int32_t whole;             // 1: every rank of an XCD runs the whole attention (see whole_call)
};

// Short contexts: a launch whose positions all lie below kWholeKeys runs, on the
// hidden-1024 bf16 body, a form of the kernel in which every workgroup of the group's XCD
// computes the group's whole attention itself (its worker waves share the positions, one
// 8-position batch each at most), so no chunk partial goes through an exchange.  A
// separate kernel, so the chunked form's code is untouched.
constexpr int kWholeKeys = 56;
inline bool whole_call(int body, int pos0, int n) { return body == BODY_Q06 && pos0 + n <= kWholeKeys; }

// Pinned id ring: the s-th id of a call goes to entry s % kIdRing as
// (call_seq << 32) | ((s / kIdRing) << 18) | id, so the host tells the entry it waits for
// from an older one (an earlier call, or an earlier lap of this call) and from a newer lap
// that has already overwritten it.  Ids are below 2^18 (the vocabulary limit) and slots
// below 2^26 (the position limit), so the lap fits its 14 bits.
constexpr int kIdRingLog2 = 12;
constexpr int kIdRing = 1 << kIdRingLog2;
__host__ __device__ inline unsigned long long ring_entry(uint32_t call_seq, int slot, int id) {
  return ((unsigned long long)call_seq << 32) | ((unsigned long long)((uint32_t)slot >> kIdRingLog2) << 18) |
         (uint32_t)(id & 0x3ffff);
}

// Tags used by one position: kPhasesPerLayer per layer plus two.  A launch also uses one
// tag (its first) for the placement check.
constexpr uint32_t kPhasesPerLayer = 8;
__host__ __device__ inline uint32_t tags_per_position(int n_layers) { return (uint32_t)n_layers * kPhasesPerLayer + 2; }

// Host-side launcher implemented next to the kernel.
int launch_decode(int body, const Params& p, bool prompt, void* stream);  // prompt: prefill_kernel
int coop_ok(int body, int* blocks_per_cu);
// The same decode as launch_decode, one kernel launch per phase (measurement only).  -2:
// the body or call has no phased form.
int launch_phased(int body, const Params& p, void* stream);
int launch_embed_sum(const void* codebooks, int n_cb, int cb_size, const void* text, int text_vocab,
                     int hidden, int bf16, const int32_t* ids, int n, float* rows, int32_t* bad, void* stream);
int launch_widen(const void* src, float* dst, int n, int bf16, void* stream);
int launch_lds_dma_selftest(const void* src, void* dst, int n_chunks, int offset_bytes, void* stream);
// Cooperative stress test of the exchange protocol (p supplies tag0, spin_limit, err, abort_flag, xq);
// local != 0: XCD-local exchanges with plain stores (place: kGrid words for the placement check).
int launch_exchange_stress(const Params& p, unsigned long long* words, unsigned long long* place, int iters, int local,
                           uint32_t* bad, void* stream);

}  // namespace mk
