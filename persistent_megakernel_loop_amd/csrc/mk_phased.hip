// Launch-per-phase decode: the persistent kernel's own phase bodies, each run as a kernel
// launch of its own.
//
// A normal (non-persistent) decode step launches the embedding lookup, the attention, the
// MLP, the norms and the sampling as separate kernels, and every launch costs time; the
// persistent kernel exists to remove that cost (the dev.to article "Porting a 1,200-line
// persistent CUDA megakernel to Qwen3-TTS", "What I took away": launch overhead is a tax
// on latency; the theaicatchup article, "Why Does a Single Kernel Even Matter for TTS?":
// hundreds of launches per forward pass).  This file measures that cost on MI355X with
// everything else held fixed: the grid (one workgroup of 512 threads per CU), the weight
// tiles and their LDS copies, the GEMV, norm, rotation, attention, combine and LM-head
// steps (mk_body.h, the same functions the persistent kernel calls, with the same
// share of every wave) and the exchange buffers and tags.  A position is 7 launches per
// layer and one for the LM head; a launch reads the words its predecessor published
// (already there when it starts, so every gather completes in its first round) and
// publishes its own.  The ids, the cache entries and the hidden states equal the
// persistent kernel's bit for bit.
//
// Measurement only: the LDS-tile bf16 bodies with one KV group per XCD (hidden <= 1024).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_body.h"
#include "mk_device.h"
#include "mk_internal.h"

namespace mk {
namespace {

enum Phase : int {
  PH_QKV = 0,   // (input or residual gather) -> input norm + q/k/v GEMV -> q/k/v rows
  PH_ATT = 1,   // q/k/v gather -> q/k norm, rotation, cache entry -> attention chunk -> chunk partial
  PH_O = 2,     // chunk gather -> combine -> O GEMV -> O partial
  PH_RES1 = 3,  // O partials of this workgroup's rows -> residual after attention
  PH_GU = 4,    // residual gather -> norm + gate/up GEMV -> SwiGLU slice
  PH_DOWN = 5,  // SwiGLU gather -> down GEMV -> down partial
  PH_RES2 = 6,  // down partials of this workgroup's rows -> residual after the MLP
  PH_LM = 7,    // residual gather -> final norm -> LM-head rows -> this workgroup's argmax key
  PH_LAST = 8,  // (one workgroup) the last position's id: outputs and the feedback id
};
constexpr int kLayerPhases = 7;
constexpr int kCtl = kWorkerWaves;  // the wave that publishes (the persistent kernel's control wave)

// Gather n (<= N) words of src that carry `tag` into dst, the eight waves taking blocks in
// turn, then a barrier.  False if the wait gave up (the timeout is recorded).
template <int N, class B>
__device__ __forceinline__ bool gather_all(const Params& P, Lds<B>& S, const u64* src, int n, uint32_t tag, float* dst,
                                           int wave, int lane) {
  constexpr int NP = kWorkerWaves + 1;
  uint32_t rounds = 0;
  unsigned long long r1 = 0;
  if (!exchange<Kp<N, NP>::value, NP>(src, n, tag, dst, 0, 0, [] {}, lane, P, rounds, r1, wave) && lane == 0)
    S.abort_ = 1;
  __syncthreads();
  return S.abort_ == 0;
}

// The copy waves copy CHUNKS 16-byte chunks into LDS and wait for them; the caller's next
// barrier publishes them to every wave.
template <int CHUNKS>
__device__ __forceinline__ void copy_tile(const uint8_t* src, void* lds, int wave, int lane) {
  dma_copy<CHUNKS>(src, lds, wave, lane);
  if (wave < kDmaWaves) wait_vmem<0>();
}

// The id position t reads (the one fed back from position t - 1 with greedy feedback);
// false if the wait for the keys gave up.
__device__ __forceinline__ bool position_id(const Params& P, int t, int lane, int* id) {
  unsigned long long ticks = 0;
  if (!P.feedback) {
    *id = P.ids[t];
    return true;
  }
  if (t == 0) {
    *id = *P.last_id;
    return true;
  }
  return argmax_keys(P, t - 1, lane, id, ticks);
}

template <class B>
__global__ void __launch_bounds__(kThreads, 1) phase_kernel(Params P, int t, int l, int phase) {
  static_assert(lds_tiles<B>() && B::BF16 && B::D == 128 && B::NG == kXcds, "LDS-tile bf16 bodies, a KV group per XCD");
  using TQKV = Tile<B, B::T_QKV, B::H>;
  using TO = Tile<B, B::T_O, B::OC>;
  using TGU = Tile<B, B::T_GU, B::H>;
  using TD = Tile<B, B::T_D, B::IX>;
  using TLM = Tile<B, 2 * kWorkerWaves, B::H>;
  constexpr int GCH = kGainFloats(B::H, B::D) * 4 / 16;
  constexpr int NC = kPerXcd * B::QPG * (B::D + 2);
  __shared__ __align__(16) u4 slotA[slot_a_bytes<B>() / 16];
  __shared__ __align__(16) u4 slotB[slot_b_bytes<B>() / 16];
  __shared__ __align__(16) Lds<B> S;
  const int b = blockIdx.x, x = b % kXcds, r = b / kXcds;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const TileAddr<B> A{P, x, r};
  const int L = P.n_layers, p = P.pos0 + t;
  const uint32_t tbase = P.tag0 + 1 + (uint32_t)t * tags_per_position(L);
  const uint32_t tg0 = tbase + (uint32_t)l * kPhasesPerLayer;
  const uint32_t tag_prev_res = tg0 - kPhasesPerLayer + 6;  // residual after the MLP of layer l - 1
  const float eps = P.rms_eps;
  float* const pp = &S.part[0][0][0];
  if (threadIdx.x == 0) S.abort_ = 0;
  __syncthreads();

  switch (phase) {
    case PH_QKV: {
      const float* gin = S.g_in0;
      if (l == 0) {
        if (wave == kCtl) {
          int id = 0;
          if (!position_id(P, t, lane, &id)) {
            if (lane == 0) S.abort_ = 1;
          } else {
            if (t > 0 && t - 1 >= P.logits_from && b == 0) {
              int prev = id;  // with feedback the fed-back id is position t - 1's
              bool ok = true;
              if (!P.feedback) {
                unsigned long long ticks = 0;
                ok = argmax_keys(P, t - 1, lane, &prev, ticks);
              }
              if (ok) publish_id(P, t - 1, prev, lane);
              else if (lane == 0) S.abort_ = 1;
            }
            input_row<B>(P, S.xs, t, id, lane);
#pragma unroll
            for (int k = 0; k < B::HPL; ++k) S.g_in0[lane + 64 * k] = P.in_norm0[lane + 64 * k];
            if (P.dbg_hidden && b == 0)
              for (int k = 0; k < B::HPL; ++k)
                P.dbg_hidden[((size_t)t * (L + 1)) * B::H + lane + 64 * k] = S.xs[lane + 64 * k];
          }
        }
      } else {
        copy_tile<GCH>(A.gains(l - 1), S.G[0], wave, lane);
        if (!gather_all<B::H>(P, S, P.xxb + (size_t)x * B::H, B::H, tag_prev_res, S.xs, wave, lane)) return;
        if (wave == kCtl && P.dbg_hidden && b == 0)
          for (int k = 0; k < B::HPL; ++k)
            P.dbg_hidden[((size_t)t * (L + 1) + l) * B::H + lane + 64 * k] = S.xs[lane + 64 * k];
        gin = S.G[0] + B::H + 2 * B::D;  // the input norm of layer l sits in layer l - 1's block
      }
      copy_tile<TQKV::TOTAL>(A.qkv(l), slotA, wave, lane);
      __syncthreads();
      if (S.abort_) return;
      tile_dot2<B::T_QKV, B::H, In::kF32Norm>(slotA, S.xs, gin, eps, S.res, wave, lane);
      __syncthreads();
      if (wave == kCtl && lane < B::T_QKV)
        st_tag(P.xq + (size_t)x * B::RQKV + r * B::T_QKV + lane, S.res[lane], tg0 + 0);
      break;
    }
    case PH_ATT: {
      copy_tile<GCH>(A.gains(l), S.G[0], wave, lane);
      if (wave == kCtl) rope_row<B>(P, S, t, p, lane);
      if (!gather_all<B::RQKV>(P, S, P.xq + (size_t)x * B::RQKV, B::RQKV, tg0 + 0, S.qkv, wave, lane)) return;
      qk_part<B>(S, S.G[0] + B::H, S.G[0] + B::H + B::D, eps, P.kv_bf16, wave, lane);
      __syncthreads();
      if (r == kPerXcd - 1 && wave == kWorkerWaves - 1) write_kv_entry<B>(P, S, x, l, p, lane);
      // the whole-attention form (P.whole): every rank of the persistent kernel runs all the
      // positions; rank 0 does it here and publishes it as the one chunk
      const int nc = P.whole ? 1 : n_chunks<B>(p);
      const int csz = (p + 1 + nc - 1) / nc;
      const bool attn = r < nc;
      const int c0 = r * csz, c1 = min(p + 1, r * csz + csz);
      if (attn && wave < kWorkerWaves) {
        KvBatch<B> unused;
        attention_chunk<B, false>(P, S, x, l, p, c0, c1, wave, lane, unused);
      }
      __syncthreads();
      if (attn && wave == kCtl) {
        float cM[B::QPG], cL[B::QPG], ca[B::QPG][B::DPL];
#pragma unroll
        for (int h = 0; h < B::QPG; ++h) {
          cM[h] = cL[h] = 0.f;
#pragma unroll
          for (int k = 0; k < B::DPL; ++k) ca[h][k] = 0.f;
        }
        merge_wave_partials<B>(S, lane, cM, cL, ca);
        u64* xa = P.xatt + (size_t)x * NC;
#pragma unroll
        for (int h = 0; h < B::QPG; ++h) {
          u64* dst = xa + ((size_t)r * B::QPG + h) * (B::D + 2);
#pragma unroll
          for (int k = 0; k < B::DPL; ++k) st_tag(dst + 2 + lane + 64 * k, ca[h][k], tg0 + 1);
          if (lane == 0) {
            st_tag(dst, cM[h], tg0 + 1);
            st_tag(dst + 1, cL[h], tg0 + 1);
          }
        }
      }
      break;
    }
    case PH_O: {
      const int nc = P.whole ? 1 : n_chunks<B>(p);
      copy_tile<TO::TOTAL>(A.o(l), slotB, wave, lane);
      if (!gather_all<NC>(P, S, P.xatt + (size_t)x * NC, nc * B::QPG * (B::D + 2), tg0 + 1, pp, wave, lane)) return;
      combine_part<B>(S, nc, wave, lane);
      __syncthreads();
      tile_dot2<B::T_O, B::OC, In::kSplit>(slotB, reinterpret_cast<const float*>(S.ov_hi),
                                           reinterpret_cast<const float*>(S.ov_lo), 0.f, S.res, wave, lane);
      __syncthreads();
      if (wave == kCtl && lane < B::T_O) st_tag(P.xop + ((size_t)r * B::NG + x) * B::T_O + lane, S.res[lane], tg0 + 2);
      break;
    }
    case PH_RES1: {
      if (!gather_all<B::NG * B::T_O>(P, S, P.xop + (size_t)r * B::NG * B::T_O, B::NG * B::T_O, tg0 + 2, pp, wave, lane))
        return;
      // this workgroup's rows of the residual before the layer
      if (l == 0) {
        if (wave == kCtl) {
          int id = 0;
          if (position_id(P, t, lane, &id)) input_row<B>(P, S.xs, t, id, lane);
          else if (lane == 0) S.abort_ = 1;
        }
        __syncthreads();
      } else if (!gather_all<B::T_O>(P, S, P.xxb + (size_t)x * B::H + r * B::T_O, B::T_O, tag_prev_res,
                                     S.xs + r * B::T_O, wave, lane)) {
        return;
      }
      if (S.abort_) return;
      if (wave == kCtl && lane < B::T_O) {
        float d = 0.f;
        for (int g = 0; g < B::NG; ++g) d += pp[g * B::T_O + lane];
        const float nv = S.xs[r * B::T_O + lane] + d;
        st_tag(P.xxa + (size_t)x * B::H + r * B::T_O + lane, nv, tg0 + 3);
      }
      break;
    }
    case PH_GU: {
      copy_tile<GCH>(A.gains(l), S.G[0], wave, lane);
      copy_tile<TGU::TOTAL>(A.gu(l), slotA, wave, lane);
      if (!gather_all<B::H>(P, S, P.xxa + (size_t)x * B::H, B::H, tg0 + 3, S.xs, wave, lane)) return;
      tile_dot2<B::T_GU, B::H, In::kF32Norm>(slotA, S.xs, S.G[0], eps, S.res, wave, lane);
      __syncthreads();
      constexpr int HALF = B::T_GU / 2;
      if (wave == kCtl && lane < HALF) {
        const float gt = S.res[lane], up = S.res[HALF + lane];
        const float mm = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
        st_tag(P.xm + (size_t)x * B::IX + r * HALF + lane, mm, tg0 + 4);
      }
      break;
    }
    case PH_DOWN: {
      copy_tile<TD::TOTAL>(A.down(l), slotB, wave, lane);
      if (!gather_all<B::IX>(P, S, P.xm + (size_t)x * B::IX, B::IX, tg0 + 4, S.mv, wave, lane)) return;
      tile_dot2<B::T_D, B::IX, In::kF32>(slotB, S.mv, nullptr, 0.f, S.res, wave, lane);
      __syncthreads();
      if (wave == kCtl && lane < B::T_D) st_tag(P.xdp + ((size_t)r * kXcds + x) * B::T_D + lane, S.res[lane], tg0 + 5);
      break;
    }
    case PH_RES2: {
      if (!gather_all<kXcds * B::T_D>(P, S, P.xdp + (size_t)r * kXcds * B::T_D, kXcds * B::T_D, tg0 + 5, pp, wave,
                                      lane))
        return;
      if (!gather_all<B::T_D>(P, S, P.xxa + (size_t)x * B::H + r * B::T_D, B::T_D, tg0 + 3, S.xs + r * B::T_D, wave,
                              lane))
        return;
      if (wave == kCtl && lane < B::T_D) {
        float d = 0.f;
        for (int g = 0; g < kXcds; ++g) d += pp[g * B::T_D + lane];
        const float nv = S.xs[r * B::T_D + lane] + d;
        st_tag(P.xxb + (size_t)x * B::H + r * B::T_D + lane, nv, tg0 + 6);
      }
      break;
    }
    case PH_LM: {  // l == L: tg0 - 8 + 6 is the last layer's residual
      const int rpb = (P.vocab + kGrid - 1) / kGrid;
      const int lm0 = b * rpb, lm1 = min(P.vocab, lm0 + rpb);
      TLM tl;
      if (wave < kWorkerWaves) lm_load<B>(tl, P, lm0, lm1, wave, lane);
      copy_tile<GCH>(A.gains(L - 1), S.G[0], wave, lane);
      if (!gather_all<B::H>(P, S, P.xxb + (size_t)x * B::H, B::H, tag_prev_res, S.xs, wave, lane)) return;
      if (wave == kCtl) {
        norm_out<B>(S.xs, S.G[0] + B::H + 2 * B::D, S.an, eps, lane);
        if (P.dbg_hidden && b == 0)
          for (int k = 0; k < B::HPL; ++k)
            P.dbg_hidden[((size_t)t * (L + 1) + L) * B::H + lane + 64 * k] = S.xs[lane + 64 * k];
      }
      __syncthreads();
      if (wave < kWorkerWaves) lm_rows<B>(P, S, tl, lm0, lm1, wave, lane);
      __syncthreads();
      if (wave == kCtl) publish_lm_key<B>(P, S, t, b, lane);
      break;
    }
    case PH_LAST: {  // grid of one workgroup: the last position's id
      if (wave == kCtl) {
        int id;
        unsigned long long ticks = 0;
        if (argmax_keys(P, t, lane, &id, ticks)) {
          publish_id(P, t, id, lane);
          if (lane == 0) *P.last_id = id;
        }
      }
      break;
    }
  }
}

template <class B>
int launch_phased_t(const Params& p, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int L = p.n_layers;
  for (int t = 0; t < p.n_pos; ++t) {
    for (int l = 0; l < L; ++l)
      for (int ph = 0; ph < kLayerPhases; ++ph)
        hipLaunchKernelGGL(phase_kernel<B>, dim3(kGrid), dim3(kThreads), 0, st, p, t, l, ph);
    hipLaunchKernelGGL(phase_kernel<B>, dim3(kGrid), dim3(kThreads), 0, st, p, t, L, (int)PH_LM);
  }
  hipLaunchKernelGGL(phase_kernel<B>, dim3(1), dim3(kThreads), 0, st, p, p.n_pos - 1, 0, (int)PH_LAST);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_phased(int body, const Params& p, void* stream) {
  if (body != BODY_Q06 || p.logits_from != 0 || p.n_pos <= 0) return -2;
  return launch_phased_t<BodyQ06>(p, stream);
}

}  // namespace mk
