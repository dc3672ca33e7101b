// Persistent batch-1 decode kernel for MI355X (gfx950, wave64).
//
// One launch runs every position of a prefill or decode call.  The op list of a
// position is the one the dev.to article ("Porting a 1,200-line persistent CUDA
// megakernel to Qwen3-TTS", section "The idea: one kernel that never exits")
// gives for a decode step -- embedding fetch, attention, MLP, norms, sampling --
// for the Qwen3 body ("Why Does a Single Kernel Even Matter for TTS?" on the
// theaicatchup article) with the talker's untied head and multi-section rotary
// embedding ("Porting it to Qwen3-TTS-1.7B").
//
// Work split (MI355X: 8 XCDs x 32 CUs, one workgroup per CU, workgroup b on XCD b%8):
//   * KV group g lives on XCD g: its q/k/v rows, its attention and the O columns
//     of its heads.  q/k/v -> attention -> O stays inside one XCD.
//   * the O projection and the down projection are split along their input
//     dimension over XCDs; each XCD publishes a partial of the whole hidden vector
//     and every workgroup sums the 8 partials of its own rows in a fixed order.
//   * the MLP slice I/8 of XCD x: gate/up rows and the matching down columns.
//   So a layer has two exchanges across XCDs and five inside an XCD.
// Exchanges are 64-bit words {value, tag}: the reader spins until every word it
// needs carries the tag of the current phase, so data and readiness travel
// together and no counter or grid barrier is needed.
//
// Workgroup: 7 worker waves stream this workgroup's weight tiles into two LDS
// slots with the LDS DMA load, a couple of exchanges before they are needed (the
// hidden-2048 body keeps them in registers instead, loaded one phase ahead), and
// do the dot products; one control wave does every exchange, so worker loads never
// sit in front of a poll in the in-order memory counter of the polling wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "mk_body.h"
#include "mk_device.h"
#include "mk_internal.h"

namespace mk {

template <class B>
__device__ __forceinline__ void worker_loop_regs(const Params& P, Lds<B>& S, int x, int r, int wave, int lane) {
  using TQKV = Tile<B, B::T_QKV, B::H>;
  using TO = Tile<B, B::T_O, B::OC>;
  using TGU = Tile<B, B::T_GU, B::H>;
  using TD = Tile<B, B::T_D, B::IX>;
  using TLM = Tile<B, 2 * kWorkerWaves, B::H>;
  constexpr int LMR = 2 * kWorkerWaves;  // LM head rows per pass
  const TileAddr<B> A{P, x, r};
  const bool grp = B::NG == kXcds || x < B::NG;
  const int L = P.n_layers;
  const int b = blockIdx.x;
  const int rpb = (P.vocab + kGrid - 1) / kGrid;
  const int lm0 = b * rpb, lm1 = min(P.vocab, lm0 + rpb);
  __builtin_assume(wave >= 0 && wave < kWorkerWaves);

  // Every load below is unconditional (addresses clamped in bounds): a conditional
  // load would make the compiler copy the registers and wait for them.  One ring streams
  // every tile: its head is loaded right after the dot product before, one exchange ahead.
  Ring q;
  TLM tl;
  // Gains block of the layer entered next, held in registers one layer ahead and
  // written to LDS (G[layer count % 2]) at that layer's first phase.
  constexpr int NT = kWorkerWaves * 64;
  constexpr int NGF = kGainFloats(B::H, B::D);
  constexpr int GPT = (NGF + NT - 1) / NT;
  const int tid = wave * 64 + lane;
  float r_g[GPT];
  auto gload = [&](int l) {
    const float* g = reinterpret_cast<const float*>(A.gains(l));
#pragma unroll
    for (int k = 0; k < GPT; ++k) r_g[k] = g[min(tid + NT * k, NGF - 1)];
  };
  int gc = 0;  // layers entered since the launch started
  // phase trace: worker wave 0 of the traced workgroup stamps, for the barrier it is about
  // to reach, when its dot product finished and when it arrived
  const bool trace = phase_traced(P, b) && wave == 0 && lane == 0;
  const int n_sync = 2 + 10 * L;
  int cur_t = 0, ph = 0;
  auto mark = [&](int k) {
    if (trace) phase_record(P, b, cur_t, n_sync, ph)[4 + k] = wall_clock64();
  };
  auto wsync = [&]() {
    mark(2);
    __syncthreads();
    ++ph;
  };
  // Waves 4..6 poll parts 1..3 of the gathers inside the XCD (the control wave polls part
  // 0); a barrier joins them.  They have no load in flight when they poll (a wave's
  // vector-memory counter is in order): they start their next tile's ring, and any other
  // load of the segment, after their part of the gather.
  const bool poller = wave >= kWorkerWaves - (kPollWaves - 1);
  // the steps after the q/k/v, attention and residual gathers, shared by the eight waves
  constexpr bool kSteps = B::BF16 && B::D == 128;
  const int part = wave - (kWorkerWaves - kPollWaves);
  const uint32_t tpp = tags_per_position(L);
  auto poll = [&](bool active, auto nmax, const u64* src, int n, uint32_t tag, float* dst, int own0, int own1) {
    constexpr int NMAX = decltype(nmax)::value;
    if (active && poller) {
      if (!help_gather<Kp<NMAX, kPollWaves>::value>(src, n, tag, dst, own0, own1, part, lane, P) && lane == 0)
        S.abort_ = 1;
      vmem_drain();
    }
  };
  auto gstore = [&]() {
    float* G = S.G[gc & 1];
#pragma unroll
    for (int k = 0; k < GPT; ++k)
      if (tid + NT * k < NGF) G[tid + NT * k] = r_g[k];
  };
  gload(0);
  stream_begin<TQKV>(q, A.qkv(0), wave, lane);

  for (int t = 0; t < P.n_pos; ++t) {
    const int p = P.pos0 + t;
    const bool lm = t >= P.logits_from;
    cur_t = t;
    ph = 0;
    const uint32_t tbase = P.tag0 + 1 + (uint32_t)t * tpp;
    wsync();  // input fetched
    if (S.abort_) return;
    auto layer = [&](int l) -> bool {
      const int ln = (l + 1 < L) ? l + 1 : 0;
      const uint32_t tg0 = tbase + (uint32_t)l * kPhasesPerLayer;
      const int nc = n_chunks<B>(p);
      const int csz = (p + 1 + nc - 1) / nc;
      const bool attn = grp && r < nc;
      const int c0 = r * csz, c1 = min(p + 1, r * csz + csz);
      // the first batch of this rank's cache rows (waves 4..6: after their part of the
      // q/k/v gather)
      KvBatch<B> kb;
      if (attn && !poller) attention_prefetch<B>(P, x, l, c0, c1, wave, lane, kb);
      // q, k, v rows
      gstore();
      if (grp) stream_dot<B, TQKV>(q, S.an, S.res, wave, lane);
      mark(1);
      if (!poller) {
        gload(ln);
        stream_begin<TO>(q, A.o(l), wave, lane);
      }
      wsync();
      poll(grp, std::integral_constant<int, B::RQKV>{}, P.xq + (size_t)x * B::RQKV, B::RQKV, tg0 + 0, S.qkv,
           r * B::T_QKV, (r + 1) * B::T_QKV);
      if (poller) {
        if (attn) attention_prefetch<B>(P, x, l, c0, c1, wave, lane, kb);
        gload(ln);
        stream_begin<TO>(q, A.o(l), wave, lane);
      }
      __syncthreads();
      if constexpr (kSteps) {
        if (grp && S.abort_ == 0) qk_part<B>(S, S.G[gc & 1] + B::H, S.G[gc & 1] + B::H + B::D, P.rms_eps, P.kv_bf16, wave, lane);
      }
      wsync();  // q rotated, k/v of position p in LDS
      if (S.abort_) return false;
      if (grp && r == kPerXcd - 1 && wave == kWorkerWaves - 1) write_kv_entry<B>(P, S, x, l, p, lane);
      // attention over this rank's chunk of positions
      if (attn) attention_chunk<B, true>(P, S, x, l, p, c0, c1, wave, lane, kb);
      wsync();
      {  // the attention chunks, polled by every wave
        constexpr int NC = kPerXcd * B::QPG * (B::D + 2);
        static_assert(comb_parts<B>() == kWorkerWaves + 1, "every wave polls the chunks");
        if (grp && !help_gather<Kp<NC, kWorkerWaves + 1>::value, kWorkerWaves + 1>(
                       P.xatt + (size_t)x * NC, nc * B::QPG * (B::D + 2), tg0 + 1, &S.part[0][0][0],
                       r < nc ? r * B::QPG * (B::D + 2) : 0, r < nc ? (r + 1) * B::QPG * (B::D + 2) : 0, wave + 1, lane,
                       P) &&
            lane == 0)
          S.abort_ = 1;
        vmem_drain();
      }
      __syncthreads();
      if constexpr (kSteps) {
        if (grp && S.abort_ == 0) combine_part<B>(S, nc, wave, lane);
      }
      wsync();  // attention output of the group in LDS
      if (S.abort_) return false;
      // O partial
      if (grp) stream_dot<B, TO>(q, S.ov, S.res, wave, lane);
      mark(1);
      if (!poller) stream_begin<TGU>(q, A.gu(l), wave, lane);
      wsync();
      poll(true, std::integral_constant<int, B::H>{}, P.xxa + (size_t)x * B::H, B::H, tg0 + 3, S.xs, r * B::T_O,
           (r + 1) * B::T_O);
      if (poller) stream_begin<TGU>(q, A.gu(l), wave, lane);
      __syncthreads();
      if constexpr (kSteps) {
        if (S.abort_ == 0) norm_out_part<B>(S.xs, S.G[gc & 1], S.an, P.rms_eps, wave, lane);
      }
      wsync();  // residual after attention, normalised
      if (S.abort_) return false;
      // gate / up
      stream_dot<B, TGU>(q, S.an, S.res, wave, lane);
      mark(1);
      if (!poller) stream_begin<TD>(q, A.down(l), wave, lane);
      wsync();
      poll(true, std::integral_constant<int, B::IX>{}, P.xm + (size_t)x * B::IX, B::IX, tg0 + 4, S.mv,
           r * (B::T_GU / 2), (r + 1) * (B::T_GU / 2));
      if (poller) stream_begin<TD>(q, A.down(l), wave, lane);
      __syncthreads();
      wsync();  // SwiGLU slice of the XCD
      if (S.abort_) return false;
      // down partial
      stream_dot<B, TD>(q, S.mv, S.res, wave, lane);
      mark(1);
      auto ahead = [&]() {
        stream_begin<TQKV>(q, A.qkv(ln), wave, lane);
      };
      if (!poller) ahead();
      wsync();
      poll(true, std::integral_constant<int, B::H>{}, P.xxb + (size_t)x * B::H, B::H, tg0 + 6, S.xs, r * B::T_D,
           (r + 1) * B::T_D);
      if (poller) ahead();
      __syncthreads();
      if constexpr (kSteps) {
        if (S.abort_ == 0) norm_out_part<B>(S.xs, S.G[gc & 1] + B::H + 2 * B::D, S.an, P.rms_eps, wave, lane);
      }
      wsync();  // residual after the MLP, normalised for the next layer or the head
      ++gc;
      return S.abort_ == 0;
    };
    for (int l = 0; l < L; ++l)
      if (!layer(l)) return;

    // LM head: this workgroup's rows, LMR per pass, two passes in flight.  Its first pass
    // is loaded here rather than during the last layer, where its 32 registers next to the
    // ring made the body spill 27 VGPRs to scratch (measured: 0.993 -> 0.923 ms/step on the
    // 1.7B talker at 512 steps once the spills were gone)
    if (lm) {
      lm_load<B>(tl, P, lm0, lm1, wave, lane);
      lm_rows<B>(P, S, tl, lm0, lm1, wave, lane);
      wsync();
    }
  }
}
// Chunk-DMA instructions wave w issues for a copy of NI instructions (none past the copy waves).
__device__ __forceinline__ constexpr int dma_count(int ni, int w) {
  return w < kDmaWaves ? (ni - w + kDmaWaves - 1) / kDmaWaves : 0;
}
// ... and for part `part` of NPARTS of it.
__device__ __forceinline__ constexpr int dma_part_count(int ni, int nparts, int part, int w) {
  return dma_count((part + 1) * ni / nparts, w) - dma_count(part * ni / nparts, w);
}

// Worker waves with the weight tiles in LDS.  Slot A holds the q/k/v tile, then gate/up;
// slot B the O tile, then down.  Each tile is copied (LDS DMA, all seven worker waves)
// as soon as its slot is free, two exchanges before its dot product, and every wave
// confirms its own copies have landed before the barrier that precedes the dot.
template <class B, bool WHOLE>
__device__ __forceinline__ void worker_loop_lds(const Params& P, Lds<B>& S, u4* slotA, u4* slotB, int x, int r, int wave,
                                int lane) {
  using TQKV = Tile<B, B::T_QKV, B::H>;
  using TO = Tile<B, B::T_O, B::OC>;
  using TGU = Tile<B, B::T_GU, B::H>;
  using TD = Tile<B, B::T_D, B::IX>;
  using TLM = Tile<B, 2 * kWorkerWaves, B::H>;
  constexpr int LMR = 2 * kWorkerWaves;
  constexpr int GCH = kGainFloats(B::H, B::D) * 4 / 16;
  static_assert(kGainFloats(B::H, B::D) % 4 == 0, "gains block in whole chunks");
  static_assert(TQKV::TOTAL * 16 <= slot_a_bytes<B>() && TGU::TOTAL * 16 <= slot_a_bytes<B>(), "slot A");
  static_assert(TO::TOTAL * 16 <= slot_b_bytes<B>() && TD::TOTAL * 16 <= slot_b_bytes<B>(), "slot B");
  // every copy writes whole 1 KB instructions: destinations must hold them
  static_assert(slot_a_bytes<B>() % 1024 == 0 && slot_b_bytes<B>() % 1024 == 0, "slots in whole KB");
  static_assert(sizeof(S.G[0]) >= (size_t)((GCH + 63) / 64) * 1024, "gains buffer in whole KB");
  constexpr int NI_Q = (TQKV::TOTAL + 63) / 64, NI_O = (TO::TOTAL + 63) / 64, NI_D = (TD::TOTAL + 63) / 64;
  constexpr int NI_GA = (GCH + 63) / 64, NI_GU = (TGU::TOTAL + 63) / 64;
  const TileAddr<B> A{P, x, r};
  const bool grp = B::NG == kXcds || x < B::NG;
  const int L = P.n_layers;
  const int b = blockIdx.x;
  const int rpb = (P.vocab + kGrid - 1) / kGrid;
  const int lm0 = b * rpb, lm1 = min(P.vocab, lm0 + rpb);
  __builtin_assume(wave >= 0 && wave < kWorkerWaves);

  // waves 4..6 poll parts 1..3 of the gathers inside the XCD (the control wave polls part 0)
  const bool poller = wave >= kWorkerWaves - (kPollWaves - 1);
  const int part = wave - (kWorkerWaves - kPollWaves);
  const uint32_t tpp = tags_per_position(L);
  // this wave's share of a gather, then the barrier that joins the gather's waves
  // (true if the gather completed everywhere: the steps after it may run)
  auto gather = [&](bool active, auto nmax, const u64* src, int n, uint32_t tag, float* dst, int own0, int own1) -> bool {
    constexpr int NMAX = decltype(nmax)::value;
    if (active && poller) {
      if (!help_gather<Kp<NMAX, kPollWaves>::value>(src, n, tag, dst, own0, own1, part, lane, P) && lane == 0)
        S.abort_ = 1;
      // An exit of the poll loop may leave a round's loads in flight.  Waiting for them
      // here, in a form the compiler sees, keeps it from waiting for them at a later merge
      // point on every wave, where the copy waves would also wait for their weight copies.
      vmem_drain();
    }
    __syncthreads();
    return active && S.abort_ == 0;
  };

  int gc = 0;  // layers entered since the launch started; gains of layer gc in G[gc % 2]
  // phase trace: worker wave 0 of the traced workgroup stamps, for the barrier it is about
  // to reach, when its copies were issued, when its dot product finished and when it arrived
  const bool trace = phase_traced(P, b) && wave == 0 && lane == 0;
  const int n_sync = 2 + 10 * L;
  int cur_t = 0, ph = 0;
  auto mark = [&](int k) {
    if (trace) phase_record(P, b, cur_t, n_sync, ph)[4 + k] = wall_clock64();
  };
  auto wsync = [&]() {
    mark(2);
    __syncthreads();
    ++ph;
  };
  dma_copy<GCH>(A.gains(0), S.G[0], wave, lane);
  dma_copy<TQKV::TOTAL>(A.qkv(0), slotA, wave, lane);
  dma_copy<TO::TOTAL>(A.o(0), slotB, wave, lane);
  wait_vmem<0>();
  TLM tl;

  for (int t = 0; t < P.n_pos; ++t) {
    const int p = P.pos0 + t;
    const bool lm = t >= P.logits_from;
    cur_t = t;
    ph = 0;
    wsync();  // input fetched
    if (S.abort_) return;
    const uint32_t tbase = P.tag0 + 1 + (uint32_t)t * tpp;
    for (int l = 0; l < L; ++l) {
      const uint32_t tg0 = tbase + (uint32_t)l * kPhasesPerLayer;
      const int ln = (l + 1 < L) ? l + 1 : 0;
      const bool lm_now = lm && l + 1 == L;
      // this rank's chunk of cache positions (all of them in the whole-attention form): its
      // first batch is loaded now
      const int nc = WHOLE ? 1 : n_chunks<B>(p);
      const int csz = (p + 1 + nc - 1) / nc;
      const bool attn = grp && (WHOLE || r < nc);
      const int c0 = WHOLE ? 0 : r * csz, c1 = WHOLE ? p + 1 : min(p + 1, r * csz + csz);
      KvBatch<B> kb;
      // (waves 4..6 load theirs after their part of the q/k/v gather: a wave's loads complete
      // in order, so rows issued here would hold back their first poll round; measured on the
      // 28-layer hidden-1024 talker: 0.3785 -> 0.3752 ms/step over 20 steps, 0.4398 -> 0.4362
      // over 256)
      if (attn && !poller) attention_prefetch<B>(P, x, l, c0, c1, wave, lane, kb);
      // this layer's O tile, behind the cache rows (slot B has been free since the last
      // down GEMV; layer 0's tile was copied before the position)
      if (l > 0) dma_copy<TO::TOTAL>(A.o(l), slotB, wave, lane);
      // Weight copies are spread over the layer's phases, about 12 KB per phase, so that
      // no exchange polls behind a large burst in this CU's memory queue: each tile is
      // copied in parts as soon as its slot is free, and waited for before the barrier
      // that precedes its dot product.
      // q, k, v rows (slot A)
      if (grp) {
        // input norm: layer 0's own gains, else the block of the layer before
        if constexpr (B::BF16)
          tile_dot2<B::T_QKV, B::H, In::kF32Norm>(slotA, S.xs, l == 0 ? S.g_in0 : S.G[(gc - 1) & 1] + B::H + 2 * B::D,
                                          P.rms_eps, S.res, wave, lane);
        else tile_dot_lds<B, TQKV>(slotA, S.an, S.res, wave, lane);
      }
      mark(1);
      wsync();
      // the q/k/v gather (as gather(), with the pollers' cache rows issued after their part)
      if (grp && poller) {
        if (!help_gather<Kp<B::RQKV, kPollWaves>::value>(P.xq + (size_t)x * B::RQKV, B::RQKV, tg0 + 0, S.qkv, r * B::T_QKV,
                                                        (r + 1) * B::T_QKV, part, lane, P) &&
            lane == 0)
          S.abort_ = 1;
        vmem_drain();
      }
      if (attn && poller) attention_prefetch<B>(P, x, l, c0, c1, wave, lane, kb);
      __syncthreads();
      if (grp && S.abort_ == 0) {
        if constexpr (B::BF16) qk_part<B>(S, S.G[gc & 1] + B::H, S.G[gc & 1] + B::H + B::D, P.rms_eps, P.kv_bf16, wave, lane);
      }
      wsync();  // q rotated, k/v of position p in LDS
      if (S.abort_) return;
      if (grp && r == kPerXcd - 1 && wave == kWorkerWaves - 1) write_kv_entry<B>(P, S, x, l, p, lane);
      // gate/up part 0 (slot A is free): issued after the q/k/v gather rather than ahead of
      // it, where it held back that gather's polls in this CU's memory queue (measured: 1 %
      // per step).  In the chunked form the copy waves' attention shares end by waiting for
      // it.  In the whole form the whole gate/up tile goes out after the attention, in one
      // burst: the compiler cannot count the copies, so the first use of the prefetched
      // cache rows waits for every load issued before it; and no exchange runs between the
      // attention and the O partials, so the burst sits ahead of no poll, while its issue
      // overlaps the control wave's merge instead of delaying the combine and the O GEMV
      // (measured on the 28-layer hidden-1024 talker: 0.3940 -> 0.3843 ms/step over 20 steps).
      if constexpr (!WHOLE) dma_part<TGU::TOTAL, 4>(A.gu(l), slotA, 0, wave, lane);
      // attention over the chunk (its cache rows were loaded at the start of the layer)
      if (attn) attention_chunk<B, true>(P, S, x, l, p, c0, c1, wave, lane, kb);
      if constexpr (WHOLE) dma_copy<TGU::TOTAL>(A.gu(l), slotA, wave, lane);
      mark(1);
      wsync();
      if constexpr (WHOLE) {
        // the whole attention in this workgroup: the control wave merges the waves' partials
        // into chunk 0 (no exchange), then every wave takes its share of the output
        if (wave < kDmaWaves) wait_vmem_rt(dma_count(NI_GU, wave));  // the O tile has landed
        mark(0);
      } else
      // the attention chunks, polled by every wave: no copy in flight (the O tile and gate/up
      // part 0 have landed), then the copy waves issue gate/up parts 1 and 2
      {
        constexpr int NC = kPerXcd * B::QPG * (B::D + 2);
        static_assert(comb_parts<B>() == kWorkerWaves + 1, "every wave polls the chunks");
        if (wave < kDmaWaves) wait_vmem<0>();
        if (grp && !help_gather<Kp<NC, kWorkerWaves + 1>::value, kWorkerWaves + 1>(
                       P.xatt + (size_t)x * NC, nc * B::QPG * (B::D + 2), tg0 + 1, &S.part[0][0][0],
                       r < nc ? r * B::QPG * (B::D + 2) : 0, r < nc ? (r + 1) * B::QPG * (B::D + 2) : 0, wave + 1, lane,
                       P) &&
            lane == 0)
          S.abort_ = 1;
        vmem_drain();
        mark(0);
        dma_part<TGU::TOTAL, 4>(A.gu(l), slotA, 1, wave, lane);
        dma_part<TGU::TOTAL, 4>(A.gu(l), slotA, 2, wave, lane);
        __syncthreads();
        if constexpr (B::BF16) {
          if (grp && S.abort_ == 0) combine_part<B>(S, nc, wave, lane);
        }
      }
      wsync();  // attention output of the group in LDS
      if (S.abort_) return;
      if constexpr (!WHOLE) dma_part<TGU::TOTAL, 4>(A.gu(l), slotA, 3, wave, lane);
      // O partial (slot B)
      if (grp) {
        if constexpr (B::BF16) tile_dot2<B::T_O, B::OC, In::kSplit>(slotB, reinterpret_cast<const float*>(S.ov_hi),
                                                              reinterpret_cast<const float*>(S.ov_lo), 0.f, S.res, wave, lane);
        else tile_dot_lds<B, TO>(slotB, S.ov, S.res, wave, lane);
      }
      mark(1);
      wsync();
      // the down tile (slot B is free) and the next layer's gains (their buffer held those
      // of the layer before this one, last read by this layer's q/k/v GEMV), issued while
      // the copy waves wait out the residual's two exchanges rather than just before the
      // gate/up GEMV, whose start their issue delayed (measured on the 28-layer hidden-1024
      // talker: 0.3972 -> 0.3938 ms/step over 20 steps, 0.4399 -> 0.4385 over 256)
      dma_part<TD::TOTAL, 2>(A.down(l), slotB, 0, wave, lane);
      dma_part<TD::TOTAL, 2>(A.down(l), slotB, 1, wave, lane);
      dma_copy<GCH>(A.gains(ln), S.G[(gc + 1) & 1], wave, lane);
      if (wave < kDmaWaves) wait_vmem_rt(dma_count(NI_D, wave) + dma_count(NI_GA, wave));  // gate/up tile landed
      gather(true, std::integral_constant<int, B::H>{}, P.xxa + (size_t)x * B::H, B::H, tg0 + 3, S.xs, r * B::T_O,
             (r + 1) * B::T_O);
      if constexpr (B::BF16) ++ph;  // residual after attention: the gather's barrier is the only one
      else wsync();               // (the fp32 body's control wave normalises after the gather)
      if (S.abort_) return;
      // gate / up (slot A)
      if constexpr (B::BF16) tile_dot2<B::T_GU, B::H, In::kF32Norm>(slotA, S.xs, S.G[gc & 1], P.rms_eps, S.res, wave, lane);
      else tile_dot_lds<B, TGU>(slotA, S.an, S.res, wave, lane);
      mark(1);
      wsync();
      if (wave < kDmaWaves) wait_vmem_rt(dma_count(NI_GA, wave));  // down tile landed
      gather(true, std::integral_constant<int, B::IX>{}, P.xm + (size_t)x * B::IX, B::IX, tg0 + 4, S.mv,
             r * (B::T_GU / 2), (r + 1) * (B::T_GU / 2));
      if constexpr (B::BF16) ++ph;  // SwiGLU slice of the XCD: the gather's barrier is the only one
      else wsync();
      if (S.abort_) return;
      dma_copy<TQKV::TOTAL>(A.qkv(ln), slotA, wave, lane);  // the next q/k/v tile: slot A is free
      // down partial (slot B)
      if constexpr (B::BF16) tile_dot2<B::T_D, B::IX, In::kF32>(slotB, S.mv, nullptr, 0.f, S.res, wave, lane);
      else tile_dot_lds<B, TD>(slotB, S.mv, S.res, wave, lane);
      mark(1);
      if (lm_now) lm_load<B>(tl, P, lm0, lm1, wave, lane);  // first LM head pass, ahead of the last exchange
      wsync();
      if (!lm_now && wave < kDmaWaves) wait_vmem<0>();  // next gains and q/k/v tile landed
      gather(true, std::integral_constant<int, B::H>{}, P.xxb + (size_t)x * B::H, B::H, tg0 + 6, S.xs, r * B::T_D,
             (r + 1) * B::T_D);
      // residual after the MLP; after the last layer a second barrier publishes the control
      // wave's final norm to the LM head
      if (!B::BF16 || l + 1 == L) wsync();
      else ++ph;
      if (!lm && l + 1 == L) dma_copy<TO::TOTAL>(A.o(0), slotB, wave, lane);  // the next position's layer 0
      ++gc;
      if (S.abort_) return;
    }
    // LM head: this workgroup's rows, LMR per pass, two passes in flight
    if (lm) {
      lm_rows<B>(P, S, tl, lm0, lm1, wave, lane);
      wait_vmem<0>();  // next gains and q/k/v tile landed
      dma_copy<TO::TOTAL>(A.o(0), slotB, wave, lane);
      wsync();
    }
  }
}

// ------------------------------------------------------------------ control wave
template <class B, bool WHOLE>
__device__ __forceinline__ void control_loop(const Params& P, Lds<B>& S, const u4* slotA, const u4* slotB, int x, int r,
                                             int lane) {
  const TileAddr<B> A{P, x, r};
  const bool grp = B::NG == kXcds || x < B::NG;
  const int L = P.n_layers;
  const int b = blockIdx.x;
  const uint32_t tpp = tags_per_position(L);
  const bool trace_phases = phase_traced(P, b);
  const int n_sync = 2 + 10 * L;  // workgroup barriers per position
  int cur_t = 0, ph = 0;
  const float eps = P.rms_eps;
  const float qscale = rsqrtf((float)B::D);
  unsigned long long wait_ticks = 0, t_start = 0;

  auto fail = [&]() { if (lane == 0) S.abort_ = 1; };
  int n_marks = 0;  // gathers completed in the current segment (first two are traced)
  // a word every lane may store to when it has nothing to publish: publishing stays branch-free
  u64* const sink = P.xsink + (size_t)b * 64 + lane;
  auto timed_exchange = [&](auto kp, auto np, const u64* src, int n, uint32_t tag, float* dst, int own0, int own1,
                            auto&& publish) {
    const unsigned long long a = wall_clock64();
    uint32_t rounds = 0;
    unsigned long long r1 = a;
    const bool ok = exchange<decltype(kp)::value, decltype(np)::value>(src, n, tag, dst, own0, own1, publish, lane, P,
                                                                       rounds, r1, 0);
    const unsigned long long e = wall_clock64();
    wait_ticks += e - a;
    if (trace_phases && lane == 0 && n_marks < 2) {
      unsigned long long* rec = phase_record(P, b, cur_t, n_sync, ph);
      rec[2 + n_marks] = e;
      // first wait: poll rounds (bits 56..63), ticks of its first round (32..55), all its ticks (0..31)
      if (n_marks == 0) rec[7] = ((u64)min(rounds, 255u) << 56) | ((u64)min(r1 - a, 0xffffffull) << 32) | (e - a);
    }
    ++n_marks;
    if (!ok) fail();
    return ok;
  };
  // A gather inside the XCD (at most NMAX words): worker waves 4..6 poll three of its four
  // parts (this wave publishes and polls part 0) and a barrier joins them (not a traced
  // phase).  `active` is uniform over the workgroup; the barrier is passed either way.
  constexpr bool kShare = true;
  constexpr int kCombParts = comb_parts<B>();
  // bf16 GEMVs with LDS tiles: this wave takes an eighth of every GEMV and of the steps after
  // the q/k/v and attention gathers; the GEMVs normalise their own inputs, so only the LM
  // head reads S.an
  constexpr bool kDots = lds_tiles<B>() && B::BF16;
  constexpr bool kNormHere = !kDots;
  // the steps after the q/k/v, attention and (register tiles) residual gathers are shared by
  // the eight waves, this one taking share 7
  constexpr bool kSteps = B::BF16 && B::D == 128;
  auto local_exchange = [&](bool active, auto nmax, const u64* src, int n, uint32_t tag, float* dst, int own0, int own1,
                            auto&& publish) -> bool {
    constexpr int NMAX = decltype(nmax)::value;
    if constexpr (kShare) {
      constexpr int NP = NMAX == kPerXcd * B::QPG * (B::D + 2) ? kCombParts : kPollWaves;
      bool ok = true;
      if (active)
        ok = timed_exchange(Kp<NMAX, NP>{}, std::integral_constant<int, NP>{}, src, n, tag, dst, own0, own1, publish);
      __syncthreads();
      return active && ok && S.abort_ == 0;
    } else {
      return active && timed_exchange(Kp<NMAX>{}, std::integral_constant<int, 1>{}, src, n, tag, dst, own0, own1, publish);
    }
  };
  // argmax over the grid's keys of the LM head that ran at position t
  auto argmax_of = [&](int t, int* out_id) -> bool {
    if (argmax_keys(P, t, lane, out_id, wait_ticks)) return true;
    fail();
    return false;
  };
  auto publish = [&](int t, int id) { publish_id(P, t, id, lane); };
  // workgroup barrier; with the phase trace on, this workgroup's arrival and departure times
  auto sync = [&]() {
    unsigned long long* rec = trace_phases ? phase_record(P, b, cur_t, n_sync, ph) : nullptr;
    if (trace_phases && lane == 0) rec[0] = wall_clock64();
    __syncthreads();
    if (trace_phases && lane == 0) rec[1] = wall_clock64();
    ++ph;
    n_marks = 0;
    return S.abort_ == 0;
  };

  int pending_lm = -1;  // position whose LM head ran and whose id is not published yet
  int gc = 0;           // layers entered since the launch started (gains in S.G[gc % 2])
  // Placement check, once per launch: every workgroup publishes the XCD it runs on.  If
  // all sit on XCD b % 8, words read only within an XCD may stay in its L2 (plain stores).
  bool lp = false;
  {
    const float* g0 = P.in_norm0;
#pragma unroll
    for (int k = 0; k < B::HPL; ++k) S.g_in0[lane + 64 * k] = g0[lane + 64 * k];
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    float* seen = &S.part[0][0][0];
    if (timed_exchange(Kp<kGrid>{}, std::integral_constant<int, 1>{}, P.xplace, kGrid, P.tag0, seen, b, b + 1, [&]() {
          st_tag(lane == 0 ? P.xplace + b : sink, __uint_as_float(xcc & 0xfu), P.tag0);
          if (lane == 0) seen[b] = __uint_as_float(xcc & 0xfu);
        })) {
      bool ok = true;
      for (int i = lane; i < kGrid; i += 64) ok &= __float_as_uint(seen[i]) == (uint32_t)(i % kXcds);
      lp = __all(ok);
    }
  }
  for (int t = 0; t < P.n_pos; ++t) {
    const int p = P.pos0 + t;
    const uint32_t tbase = P.tag0 + 1 + (uint32_t)t * tpp;
    cur_t = t;
    ph = 0;
    t_start = wall_clock64();
    wait_ticks = 0;
    // ---------------------------------------------------------------- input of position t
    {
      int id = 0;
      bool ok = true;
      if (P.feedback) {
        if (t == 0) id = *P.last_id;
        else ok = argmax_of(t - 1, &id);
        if (ok && t > 0 && b == 0) publish(t - 1, id);
        pending_lm = -1;
      } else {
        id = P.ids[t];
        if (pending_lm >= 0 && b == 0) {
          int pid;
          if ((ok = argmax_of(pending_lm, &pid))) publish(pending_lm, pid);
        }
        pending_lm = -1;
      }
      if (ok) {
        input_row<B>(P, S.xs, t, id, lane);
        rope_row<B>(P, S, t, p, lane);
        if constexpr (kNormHere) {
          if constexpr (B::BF16) norm_out<B>(S.xs, S.g_in0, S.an, eps, lane);
          else norm_to<B>(S.xs, S.g_in0, S.an, eps, lane);
        }
        if (P.dbg_hidden && b == 0)
          for (int k = 0; k < B::HPL; ++k)
            P.dbg_hidden[((size_t)t * (L + 1)) * B::H + lane + 64 * k] = S.xs[lane + 64 * k];
      }
    }
    if (!sync()) return;

    for (int l = 0; l < L; ++l) {
      const uint32_t tg0 = tbase + (uint32_t)l * kPhasesPerLayer;
      // this wave's share of the bf16 GEMVs with tiles in LDS (the eighth row block)
      if constexpr (kDots) {
        if (grp)
          tile_dot2<B::T_QKV, B::H, In::kF32Norm>(slotA, S.xs, l == 0 ? S.g_in0 : S.G[(gc - 1) & 1] + B::H + 2 * B::D, eps, S.res,
                                          kWorkerWaves, lane);
      }
      // ------------------------------------------------------------ q,k,v of the group
      if (!sync()) return;
      {
        u64* xq = P.xq + (size_t)x * B::RQKV;
        if (local_exchange(grp, std::integral_constant<int, B::RQKV>{}, xq, B::RQKV, tg0 + 0, S.qkv, r * B::T_QKV,
                           (r + 1) * B::T_QKV, [&]() {
              st_local(lane < B::T_QKV ? xq + r * B::T_QKV + lane : sink, S.res[lane], tg0 + 0, lp);
              if (lane < B::T_QKV) S.qkv[r * B::T_QKV + lane] = S.res[lane];
            })) {
          // per-head RMSNorm of q and k, rotation, rounding of the cache entry
          const float* qn = S.G[gc & 1] + B::H;
          const float* kn = S.G[gc & 1] + B::H + B::D;
          if constexpr (kSteps) {
            qk_part<B>(S, qn, kn, eps, P.kv_bf16, kWorkerWaves, lane);  // waves 0..3 take the heads
          } else if constexpr (B::D == 128) {
            // lane i holds elements i and i + 64 of every head, which are rotary pair i:
            // norm and rotation stay in registers, the q heads and k side by side
            const float c = S.rope_c[lane], sn = S.rope_s[lane];
            float a0[B::QPG + 1], a1[B::QPG + 1], ss[B::QPG + 1];
#pragma unroll
            for (int h = 0; h <= B::QPG; ++h) {
              a0[h] = S.qkv[h * B::D + lane];
              a1[h] = S.qkv[h * B::D + lane + 64];
              ss[h] = fmaf(a1[h], a1[h], a0[h] * a0[h]);
            }
#pragma unroll
            for (int h = 0; h <= B::QPG; ++h) ss[h] = wave_sum(ss[h]);
            const float vv0 = S.qkv[(B::QPG + 1) * B::D + lane], vv1 = S.qkv[(B::QPG + 1) * B::D + lane + 64];
#pragma unroll
            for (int h = 0; h <= B::QPG; ++h) {
              const float* g = h < B::QPG ? qn : kn;
              const float rs = __builtin_amdgcn_rsqf(ss[h] / (float)B::D + eps);
              const float n0 = g[lane] * (a0[h] * rs), n1 = g[lane + 64] * (a1[h] * rs);
              float o0 = n0 * c - n1 * sn, o1 = n1 * c + n0 * sn;
              if (h < B::QPG) {
                S.qkv[h * B::D + lane] = o0 * qscale;
                S.qkv[h * B::D + lane + 64] = o1 * qscale;
              } else {
                if (P.kv_bf16) { o0 = bf16_round(o0); o1 = bf16_round(o1); }
                S.kp[lane] = o0;
                S.kp[lane + 64] = o1;
              }
            }
            S.vp[lane] = P.kv_bf16 ? bf16_round(vv0) : vv0;
            S.vp[lane + 64] = P.kv_bf16 ? bf16_round(vv1) : vv1;
          } else for (int h = 0; h <= B::QPG; ++h) {  // h == QPG is k
            float* v = S.qkv + h * B::D;
            const float* g = h < B::QPG ? qn : kn;
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) { const float a = v[lane + 64 * k]; ss = fmaf(a, a, ss); }
            ss = wave_sum(ss);
            const float rs = __builtin_amdgcn_rsqf(ss / (float)B::D + eps);
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) { const int i = lane + 64 * k; v[i] = g[i] * (v[i] * rs); }
            // LDS accesses of one wave are performed in order: the lane owning pair i
            // sees every lane's normalised value
            for (int i = lane; i < B::D / 2; i += 64) {
              const float c = S.rope_c[i];
              const float sn = S.rope_s[i];
              const float a0 = v[i], a1 = v[i + B::D / 2];
              float o0 = a0 * c - a1 * sn, o1 = a1 * c + a0 * sn;
              if (h < B::QPG) {
                v[i] = o0 * qscale;
                v[i + B::D / 2] = o1 * qscale;
              } else {
                if (P.kv_bf16) { o0 = bf16_round(o0); o1 = bf16_round(o1); }
                S.kp[i] = o0;
                S.kp[i + B::D / 2] = o1;
              }
            }
          }
          if constexpr (B::D != 128) {
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) {
              const int i = lane + 64 * k;
              const float v = S.qkv[(B::QPG + 1) * B::D + i];
              S.vp[i] = P.kv_bf16 ? bf16_round(v) : v;
            }
          }
        }
      }
      if (!sync()) return;
      // ------------------------------------------------------------ attention combine
      if (!sync()) return;
      if constexpr (WHOLE) {
        // every rank ran the whole attention: its waves' partials merged are the result.
        // This wave also finishes it, with no second barrier: the combine of one chunk
        // (weight exactly 1, sum exactly its L) in the same operations, so the output
        // equals the chunked form's bit for bit, then the split for the O GEMV.
        float cM[B::QPG], cL[B::QPG], ca[B::QPG][B::DPL];
#pragma unroll
        for (int h = 0; h < B::QPG; ++h) {
          cM[h] = cL[h] = 0.f;
#pragma unroll
          for (int k = 0; k < B::DPL; ++k) ca[h][k] = 0.f;
        }
        if (grp) {
          merge_wave_partials<B>(S, lane, cM, cL, ca);
#pragma unroll
          for (int h = 0; h < B::QPG; ++h) {
            const float inv = __builtin_amdgcn_rcpf(cL[h]);
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) S.ov[h * B::D + lane + 64 * k] = fmaf(ca[h][k], 1.f, 0.f) * inv;
          }
          // (this wave's own LDS writes are seen by its later reads)
          static_assert(B::OC / 8 <= 64, "a chunk per lane");
          if (lane < B::OC / 8) split8(S.ov + 8 * lane, S.ov_hi[lane], S.ov_lo[lane]);
        }
      } else {
        const int nc = n_chunks<B>(p);
        u64* xa = P.xatt + (size_t)x * kPerXcd * B::QPG * (B::D + 2);
        // this rank's chunk partial: the worker waves' partials merged in a fixed order
        float cM[B::QPG], cL[B::QPG], ca[B::QPG][B::DPL];
#pragma unroll
        for (int h = 0; h < B::QPG; ++h) {
          cM[h] = cL[h] = 0.f;
#pragma unroll
          for (int k = 0; k < B::DPL; ++k) ca[h][k] = 0.f;
        }
        if (grp && r < nc) merge_wave_partials<B>(S, lane, cM, cL, ca);
        auto publish_chunk = [&]() {  // ranks without a chunk store to the sink
          const bool mine = r < nc;
#pragma unroll
          for (int h = 0; h < B::QPG; ++h) {
            u64* dst = xa + ((size_t)(mine ? r : 0) * B::QPG + h) * (B::D + 2);
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) {
              st_local(mine ? dst + 2 + lane + 64 * k : sink, ca[h][k], tg0 + 1, lp);
              if (mine) S.part[r][h][2 + lane + 64 * k] = ca[h][k];
            }
            st_local(mine && lane == 0 ? dst : sink, cM[h], tg0 + 1, lp);
            st_local(mine && lane == 0 ? dst + 1 : sink, cL[h], tg0 + 1, lp);
            if (mine && lane == 0) {
              S.part[r][h][0] = cM[h];
              S.part[r][h][1] = cL[h];
            }
          }
        };
        const int own0 = r < nc ? r * B::QPG * (B::D + 2) : 0, own1 = r < nc ? (r + 1) * B::QPG * (B::D + 2) : 0;
        const bool got = local_exchange(grp, std::integral_constant<int, kPerXcd * B::QPG * (B::D + 2)>{}, xa,
                                        nc * B::QPG * (B::D + 2), tg0 + 1, &S.part[0][0][0], own0, own1, publish_chunk);
        if constexpr (kSteps) {
          if (got) combine_part<B>(S, nc, kWorkerWaves, lane);
        } else if (got) {
          // chunks four at a time: their loads are independent (chunks past nc weigh 0)
#pragma unroll
          for (int h = 0; h < B::QPG; ++h) {
            float M = -INFINITY;
            for (int c0 = 0; c0 < nc; c0 += 4) {
#pragma unroll
              for (int c = c0; c < c0 + 4; ++c) M = fmaxf(M, c < nc ? S.part[c][h][0] : -INFINITY);
            }
            float Ls = 0.f, a[B::DPL];
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) a[k] = 0.f;
            for (int c0 = 0; c0 < nc; c0 += 4) {
#pragma unroll
              for (int c = c0; c < c0 + 4; ++c) {
                const int cc = min(c, nc - 1);
                const float mc = S.part[cc][h][0];
                const float f = (c < nc && mc != -INFINITY) ? __expf(mc - M) : 0.f;
                Ls = fmaf(S.part[cc][h][1], f, Ls);
#pragma unroll
                for (int k = 0; k < B::DPL; ++k) a[k] = fmaf(S.part[cc][h][2 + lane + 64 * k], f, a[k]);
              }
            }
            const float inv = __builtin_amdgcn_rcpf(Ls);
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) S.ov[h * B::D + lane + 64 * k] = a[k] * inv;
          }
        }
      }
      if (!sync()) return;
      // ------------------------------------------------------------ O partials -> residual
      if constexpr (kDots) {
        if (grp) tile_dot2<B::T_O, B::OC, In::kSplit>(slotB, reinterpret_cast<const float*>(S.ov_hi),
                                                       reinterpret_cast<const float*>(S.ov_lo), 0.f, S.res, kWorkerWaves, lane);
      }
      if (!sync()) return;
      {
        // group x's partial of rows [r*T_O, (r+1)*T_O) goes to slot [r][x]: the reader of
        // those rows finds every group's partial in one contiguous run
        float* pp = &S.part[0][0][0];
        // this XCD's rows of the residual: every group's partial (across the XCDs)
        const bool got = timed_exchange(Kp<B::NG * B::T_O>{}, std::integral_constant<int, 1>{},
                                        P.xop + (size_t)r * B::NG * B::T_O, B::NG * B::T_O, tg0 + 2, pp,
                                        grp ? x * B::T_O : 0, grp ? (x + 1) * B::T_O : 0, [&]() {
                                          const bool mine = grp && lane < B::T_O;
                                          st_tag(mine ? P.xop + ((size_t)r * B::NG + x) * B::T_O + lane : sink, S.res[lane],
                                                 tg0 + 2);
                                          if (mine) pp[x * B::T_O + lane] = S.res[lane];
                                        });
        float nv = 0.f;
        if (got && lane < B::T_O) {
          float d = 0.f;
          for (int g = 0; g < B::NG; ++g) d += pp[g * B::T_O + lane];
          nv = S.xs[r * B::T_O + lane] + d;
        }
        // then the whole residual inside the XCD
        if (local_exchange(got, std::integral_constant<int, B::H>{}, P.xxa + (size_t)x * B::H, B::H, tg0 + 3, S.xs,
                           r * B::T_O, (r + 1) * B::T_O, [&]() {
                             st_local(lane < B::T_O ? P.xxa + (size_t)x * B::H + r * B::T_O + lane : sink, nv, tg0 + 3, lp);
                             if (lane < B::T_O) S.xs[r * B::T_O + lane] = nv;
                           })) {
          if constexpr (kSteps && kNormHere) {
            norm_out_part<B>(S.xs, S.G[gc & 1], S.an, eps, kWorkerWaves, lane);
          } else if constexpr (kNormHere) {
            if constexpr (B::BF16) norm_out<B>(S.xs, S.G[gc & 1], S.an, eps, lane);
            else norm_to<B>(S.xs, S.G[gc & 1], S.an, eps, lane);
          }
        }
      }
      if constexpr (kDots) {  // nothing since the gather's barrier: no second one
        ++ph;
        n_marks = 0;
        if (S.abort_) return;
      } else if (!sync()) {
        return;
      }
      // ------------------------------------------------------------ SwiGLU slice
      if constexpr (kDots) tile_dot2<B::T_GU, B::H, In::kF32Norm>(slotA, S.xs, S.G[gc & 1], eps, S.res, kWorkerWaves, lane);
      if (!sync()) return;
      {
        constexpr int HALF = B::T_GU / 2;
        float mm = 0.f;
        if (lane < HALF) {
          const float gt = S.res[lane], up = S.res[HALF + lane];
          mm = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
        }
        local_exchange(true, std::integral_constant<int, B::IX>{}, P.xm + (size_t)x * B::IX, B::IX, tg0 + 4, S.mv, r * HALF,
                       (r + 1) * HALF, [&]() {
                         st_local(lane < HALF ? P.xm + (size_t)x * B::IX + r * HALF + lane : sink, mm, tg0 + 4, lp);
                         if (lane < HALF) S.mv[r * HALF + lane] = mm;
                       });
      }
      if constexpr (kDots) {  // nothing since the gather's barrier: no second one
        ++ph;
        n_marks = 0;
        if (S.abort_) return;
      } else if (!sync()) {
        return;
      }
      // ------------------------------------------------------------ down partials -> residual
      if constexpr (kDots) tile_dot2<B::T_D, B::IX, In::kF32>(slotB, S.mv, nullptr, 0.f, S.res, kWorkerWaves, lane);
      if (!sync()) return;
      {
        float* pp = &S.part[0][0][0];
        const bool got = timed_exchange(Kp<kXcds * B::T_D>{}, std::integral_constant<int, 1>{},
                                        P.xdp + (size_t)r * kXcds * B::T_D, kXcds * B::T_D, tg0 + 5, pp, x * B::T_D,
                                        (x + 1) * B::T_D, [&]() {
                                          st_tag(lane < B::T_D ? P.xdp + ((size_t)r * kXcds + x) * B::T_D + lane : sink,
                                                 S.res[lane], tg0 + 5);
                                          if (lane < B::T_D) pp[x * B::T_D + lane] = S.res[lane];
                                        });
        float nv = 0.f;
        if (got && lane < B::T_D) {
          float d = 0.f;
          for (int g = 0; g < kXcds; ++g) d += pp[g * B::T_D + lane];
          nv = S.xs[r * B::T_D + lane] + d;
        }
        if (local_exchange(got, std::integral_constant<int, B::H>{}, P.xxb + (size_t)x * B::H, B::H, tg0 + 6, S.xs,
                           r * B::T_D, (r + 1) * B::T_D, [&]() {
                             st_local(lane < B::T_D ? P.xxb + (size_t)x * B::H + r * B::T_D + lane : sink, nv, tg0 + 6, lp);
                             if (lane < B::T_D) S.xs[r * B::T_D + lane] = nv;
                           })) {
          // the next layer's input norm, or the final norm ahead of the LM head
          if constexpr (kSteps && kNormHere) {
            norm_out_part<B>(S.xs, S.G[gc & 1] + B::H + 2 * B::D, S.an, eps, kWorkerWaves, lane);
          } else if (kNormHere || l + 1 == L) {
            if constexpr (B::BF16) norm_out<B>(S.xs, S.G[gc & 1] + B::H + 2 * B::D, S.an, eps, lane);
            else norm_to<B>(S.xs, S.G[gc & 1] + B::H + 2 * B::D, S.an, eps, lane);
          }
          if (P.dbg_hidden && b == 0)
            for (int k = 0; k < B::HPL; ++k)
              P.dbg_hidden[((size_t)t * (L + 1) + l + 1) * B::H + lane + 64 * k] = S.xs[lane + 64 * k];
        }
      }
      ++gc;
      if (!kDots || l + 1 == L) {
        if (!sync()) return;
      } else {  // nothing since the gather's barrier: no second one
        ++ph;
        n_marks = 0;
        if (S.abort_) return;
      }
    }  // layers

    // ---------------------------------------------------------------- argmax key of this workgroup
    if (t >= P.logits_from) {
      sync();  // workers' per-wave best
      publish_lm_key<B>(P, S, t, b, lane);
      pending_lm = t;
    }
    if (P.dbg_trace && lane == 0) {
      P.dbg_trace[((size_t)t * kGrid + b) * 2 + 0] = wait_ticks;
      P.dbg_trace[((size_t)t * kGrid + b) * 2 + 1] = wall_clock64() - t_start;
    }
  }  // positions

  // publish the last id and keep it for feedback
  if (b == 0 && pending_lm >= 0) {
    int id;
    if (argmax_of(pending_lm, &id)) {
      publish(pending_lm, id);
      if (lane == 0) *P.last_id = id;
    }
  }
}

template <class B, bool WHOLE>
__device__ __forceinline__ void persistent_body(const Params& P) {
  __shared__ __align__(16) u4 slotA[slot_a_bytes<B>() / 16];
  __shared__ __align__(16) u4 slotB[slot_b_bytes<B>() / 16];
  __shared__ __align__(16) Lds<B> S;
  const int b = blockIdx.x, x = b % kXcds, r = b / kXcds;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (threadIdx.x == 0) S.abort_ = 0;
  if (wave == kWorkerWaves) control_loop<B, WHOLE>(P, S, slotA, slotB, x, r, lane);
  else if constexpr (lds_tiles<B>()) worker_loop_lds<B, WHOLE>(P, S, slotA, slotB, x, r, wave, lane);
  else worker_loop_regs<B>(P, S, x, r, wave, lane);
}

// The same persistent body under two names, so that a profile tells decode launches
// (the LM head at every step) from prompt launches (the LM head at the last position).
template <class B, bool WHOLE>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(Params P) { persistent_body<B, WHOLE>(P); }
template <class B, bool WHOLE>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(Params P) { persistent_body<B, WHOLE>(P); }

// Bodies with a whole-attention form (whole_call).
template <class B>
constexpr bool has_whole() { return lds_tiles<B>() && B::BF16 && B::D == 128; }

// Dynamic LDS added to the kernel's static LDS so that a workgroup takes more than half
// of a CU's 160 KB: the grid then places exactly one workgroup on each CU.
template <class B>
static int lds_padding() {
  hipFuncAttributes a;
  if (hipFuncGetAttributes(&a, (const void*)decode_kernel<B, false>) != hipSuccess) return -1;
  const int need = 80 * 1024 + 1024 - (int)a.sharedSizeBytes;
  return need > 0 ? need : 0;
}

template <class B>
static int launch_t(const Params& p, bool prompt, void* stream) {
  Params pp = p;
  void* args[] = {&pp};
  const int pad = lds_padding<B>();
  if (pad < 0) return -1;
  const void* fn = prompt ? (const void*)prefill_kernel<B, false> : (const void*)decode_kernel<B, false>;
  if constexpr (has_whole<B>()) {
    if (p.whole) fn = prompt ? (const void*)prefill_kernel<B, true> : (const void*)decode_kernel<B, true>;
  } else if (p.whole) {
    return -1;
  }
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(kGrid), dim3(kThreads), args, (unsigned)pad, (hipStream_t)stream);
  return e == hipSuccess ? 0 : -1;
}

template <class B>
static int coop_t(int* blocks) {
  const int pad = lds_padding<B>();
  if (pad < 0) return -1;
  int nb[4] = {0, 0, 0, 0};
  const void* fns[4] = {(const void*)decode_kernel<B, false>, (const void*)prefill_kernel<B, false>, nullptr, nullptr};
  if constexpr (has_whole<B>()) {
    fns[2] = (const void*)decode_kernel<B, true>;
    fns[3] = (const void*)prefill_kernel<B, true>;
  }
  int best = 1 << 30;
  for (int k = 0; k < 4; ++k) {
    if (!fns[k]) continue;
    if (pad > 0 && hipFuncSetAttribute(fns[k], hipFuncAttributeMaxDynamicSharedMemorySize, pad) != hipSuccess) return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb[k], fns[k], kThreads, pad) != hipSuccess) return -1;
    best = nb[k] < best ? nb[k] : best;
  }
  *blocks = best;
  return 0;
}

int launch_decode(int body, const Params& p, bool prompt, void* stream) {
  switch (body) {
    case BODY_TINY: return launch_t<BodyTiny>(p, prompt, stream);
    case BODY_Q06: return launch_t<BodyQ06>(p, prompt, stream);
    case BODY_Q17: return launch_t<BodyQ17>(p, prompt, stream);
  }
  return -1;
}

int coop_ok(int body, int* blocks) {
  switch (body) {
    case BODY_TINY: return coop_t<BodyTiny>(blocks);
    case BODY_Q06: return coop_t<BodyQ06>(blocks);
    case BODY_Q17: return coop_t<BodyQ17>(blocks);
  }
  return -1;
}

}  // namespace mk
