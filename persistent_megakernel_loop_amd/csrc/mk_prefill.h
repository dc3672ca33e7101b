// Internal declarations of the batched prompt prefill (host library side).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "mk_internal.h"

namespace mk {

// Batched prompt prefill (all prompt positions but the last, in chunks of up to
// kPrefillChunk positions): arguments of one chunk.
constexpr int kPrefillChunk = 64;
struct PfArgs {
  int32_t H, D, NQ, NKV, I, L, vocab, max_seq, rope_positions;
  int32_t n_sections, sec_end0, sec_end1;
  float eps;
  int32_t kv_bf16;
  const uint16_t* embed;     // [V][H] bf16
  const float* in_norm0;     // [H]
  const float* rope_cos;     // [rope_positions][D/2]
  const float* rope_sin;
  void* kcache;              // [L][NKV][max_seq][D]
  void* vcache;
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
};
size_t prefill_part_floats(int H, int NQ, int NKV, int D, int I);  // 0: shape not supported
int launch_prefill_chunk(const PfArgs& a, const uint8_t* layers, const LayerLayout& lay, void* stream);
int launch_gemm_selftest(const uint16_t* w, int R, int K, const float* x, int m, float* y, uint16_t* xs, float* part,
                         void* stream);

}  // namespace mk
