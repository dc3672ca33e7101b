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
int launch_prefill_lm(const PfArgs& a, const LmArgs& lm, void* stream);
int launch_prefill_chunk(const PfArgs& a, const uint8_t* layers, const LayerLayout& lay, void* stream);
// Read-stream ceiling (a measurement kernel, not part of the decode path).
int launch_stream_read(const void* src, size_t bytes, int nontemporal, unsigned long long* sink, int blocks,
                       void* stream);
int launch_gemm_selftest(const uint16_t* w, int R, int K, const float* x, int m, float* y, uint16_t* xs, float* part,
                         void* stream);

}  // namespace mk
