// Internal declarations of the batched prompt prefill (host library side).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "mk_internal.h"

namespace mk {

// Batched prompt prefill (every prompt position, in chunks of up to kPrefillChunk
// positions): arguments of one chunk.
constexpr int kPrefillChunk = 64;
constexpr int kFlashRanges = 64;  // key ranges of the prefill attention, at most
struct PfArgs {
  int32_t H, D, NQ, NKV, I, L, vocab, max_seq, rope_positions;
  int32_t n_sections, sec_end0, sec_end1;
  float eps;
  const uint16_t* embed;     // [V][H] bf16
  const float* in_norm0;     // [H]
  const float* rope_cos;     // [rope_positions][D/2]
  const float* rope_sin;
  uint16_t* kcache;          // [L][NKV][max_seq][D] bf16 (the batched path serves bf16 bodies, whose cache is bf16)
  uint16_t* vcache;
  uint32_t* err;             // device error word
  int32_t m;                 // positions in the chunk
  int32_t npp;               // columns of the products: m rounded up to a multiple of 16
  int32_t pos0;              // position of the chunk's first row
  const int32_t* ids;        // [m], the chunk's first entry
  const float* rows;         // [m][H] or NULL
  const int32_t* pos3;       // [m][3] or NULL
  float* dbg_hidden;         // [m][L+1][H] or NULL
  float* x;                  // [npp][H] residual stream
  uint16_t* xs;              // [2][K/8][npp][8] split activations, K up to max(H, NQ*D, I)
  float* part;               // partial products, prefill_part_floats() floats
  float* q;                  // [npp][NQ][D] rotated, scaled queries
  float* att;                // [NKV][kFlashRanges][2 npp rows][D + 2] attention partials (max, sum, output)
  float* ss;                 // [npp][H/512] sums of squares of the residual row, per 512 columns
};
// The prompt's first id: the LM head over the last prompt position's final-norm row,
// greedy (ties: lowest index), published like a decode step's id.
constexpr int kLmRowsPerBlock = 64;
struct LmArgs {
  const uint16_t* lm_head;   // [V][H] bf16
  const float* g_final;      // [H] final norm gains
  int32_t n_last;            // row of the last position in the chunk's residual stream
  float* blk_val;            // [ceil(V / kLmRowsPerBlock)] per-block maxima
  int32_t* blk_idx;
  int32_t* out_first;        // [1] device
  int32_t* last_id;          // feedback id for the next decode call
  unsigned long long* pinned_ids;  // host-pinned id ring (ring_entry), or NULL
  unsigned long long* progress;  // host-pinned progress word
  uint32_t call_seq;
};
size_t prefill_part_floats(int H, int NQ, int NKV, int D, int I);  // 0: shape not supported

// The same chunk as one persistent launch (mk_pprefill.hip): every workgroup stays
// resident for all layers and the phases hand over through flagged buffers instead of
// kernel boundaries.  Hidden 1024, intermediate 3072, head_dim 128, 16 query and 8 KV
// heads (the hidden-1024 talker and text bodies), chunks whose context ends at or below
// kPpMaxKeys.  Exchange regions, per XCD replica where marked; NPP is the chunk's column
// count (a multiple of 16, at most kPrefillChunk):
constexpr int kPpMaxKeys = 2048;
constexpr int kPpKinds = 8;  // flag words per workgroup: one per hand-over kind
struct PpBufs {
  unsigned long long* flags;  // [kPpKinds][kGrid] tagged words {0, tag}, zero before the first use
  uint16_t* xb;  // [8][2][H/8][NPP][8] bf16 high, then low parts: input-norm gains * x, the q/k/v operand
  uint16_t* xp;  // [8][2][H/8][NPP][8] post-attention-norm gains * x, the gate/up operand
  float* ss;     // [8][32][NPP] sums of squares of x over each owner's 32 columns (input norm)
  float* ss2;    // [8][32][NPP] the same after attention
  float* qr;     // [8][NPP][512] q/k/v of the group, times the input norm's 1/rms
  uint16_t* at;  // [8][2][32][NPP][8] attention outputs of the group, split, the O operand
  float* op;     // [8 XCDs][32][NPP][32] O partials of each XCD's KV block, by owner
  uint16_t* hs;  // [8][2][48][NPP][8] SwiGLU outputs of the XCD's MLP slice, split, the down operand
  float* dp;     // [8][32][NPP][32] down partials of each XCD's MLP slice, by owner
};
// Byte offsets of the regions above (relative to a base) for chunks of up to
// kPrefillChunk positions; returns the total.  0: the shape has no persistent form.
size_t pp_layout(int H, int NQ, int NKV, int D, int I, size_t offs[10]);
// The chunk in A, layer weights at `layers`: every layer of the chunk, leaving the final
// residual of its positions in A.x for launch_prefill_lm.  tag0: first of the
// (L + 1) * 8 flag tags this launch uses, all above any tag the flag words hold.
// dbg_phase, if not NULL, receives [grid][L + 1][kPpKinds][2] 100 MHz ticks: for each
// hand-over kind produced in layer l (slot l + 1; slot 0: the input rows and the launch's
// placement check), when the workgroup's wait for it completed and when it raised its
// own flag of that kind.
int launch_prefill_persistent(const PfArgs& A, const PpBufs& B, const uint8_t* layers, const LayerLayout& lay,
                              uint32_t tag0, uint32_t spin_limit, uint32_t* abort_flag, unsigned long long* dbg_phase,
                              void* stream);
bool pp_supported(int H, int NQ, int NKV, int D, int I);
// Zeroes the kPpKinds * kGrid flag words (a kernel, so the call may sit in a captured graph).
int launch_pp_clear(unsigned long long* flags, void* stream);
int launch_prefill_lm(const PfArgs& a, const LmArgs& lm, void* stream);
int launch_prefill_chunk(const PfArgs& a, const uint8_t* layers, const LayerLayout& lay, void* stream);
// Read-stream ceiling (a measurement kernel, not part of the decode path).
int launch_stream_read(const void* src, size_t bytes, int nontemporal, unsigned long long* sink, int blocks,
                       void* stream);
int launch_gemm_selftest(const uint16_t* w, int R, int K, const float* x, int m, float* y, uint16_t* xs, float* part,
                         void* stream);

}  // namespace mk
