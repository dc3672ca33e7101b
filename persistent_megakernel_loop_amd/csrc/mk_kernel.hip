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

#include "mk_device.h"
#include "mk_internal.h"

namespace mk {


// ------------------------------------------------------------------ body shapes
template <int H_, int D_, int NQ_, int NKV_, int I_, bool BF16_>
struct Body {
  static constexpr int H = H_, D = D_, NQ = NQ_, NKV = NKV_, I = I_;
  static constexpr bool BF16 = BF16_;
  static constexpr int E = BF16 ? 8 : 4;       // weights per 16-byte chunk
  static constexpr int WB = BF16 ? 2 : 4;      // bytes per weight
  static constexpr int NG = NKV;               // XCDs that own a KV group
  static constexpr int QPG = NQ / NKV;         // query heads per group
  static constexpr int RQKV = (QPG + 2) * D;   // q,k,v rows of one group
  static constexpr int OC = QPG * D;           // O input columns of one group
  static constexpr int IX = I / kXcds;         // MLP slice of one XCD
  static constexpr int T_QKV = RQKV / kPerXcd; // rows per workgroup tile
  static constexpr int T_O = H / kPerXcd;
  static constexpr int T_GU = 2 * IX / kPerXcd;
  static constexpr int T_D = H / kPerXcd;
  static constexpr int DPL = D / 64;           // head dims per lane (attention, rotation)
  static constexpr int HPL = H / 64;           // hidden elements per lane
  static_assert(NKV <= kXcds && kXcds % NKV == 0, "one KV group per XCD");
  static_assert(NQ % NKV == 0, "GQA");
  static_assert(RQKV % kPerXcd == 0 && H % (kPerXcd * 2) == 0 && (2 * IX) % kPerXcd == 0, "tiles");
  static_assert(D % 64 == 0 && H % 64 == 0, "lanes");
};
using BodyTiny = Body<256, 64, 4, 2, 768, false>;
using BodyQ06 = Body<1024, 128, 16, 8, 3072, true>;
using BodyQ17 = Body<2048, 128, 16, 8, 6144, true>;

// A weight tile: ROWS consecutive rows of COLS columns, contiguous in the arena.
// Worker wave w < NWA owns rows [w*RPW, (w+1)*RPW) (the last wave may own fewer):
// chunks w*CPW .. w*CPW+CPW-1 of the tile, read lane-linearly, 16 bytes per lane.
template <class B, int ROWS, int COLS>
struct Tile {
  static constexpr int NWA = ROWS < kWorkerWaves ? ROWS : kWorkerWaves;
  static constexpr int RPW = (ROWS + NWA - 1) / NWA;
  static constexpr int CPR = COLS / B::E;
  static constexpr int CPW = RPW * CPR;
  static constexpr int TOTAL = ROWS * CPR;     // chunks in the tile
  static constexpr int LPL = (CPW + 63) / 64;
  static constexpr bool EXACT = CPW % 64 == 0 && NWA * CPW == TOTAL;  // no chunk needs a guard
  static constexpr size_t BYTES = (size_t)ROWS * COLS * B::WB;
  static_assert(COLS % B::E == 0, "chunk");
  u4 v[LPL];
};

// Waves that poll the gathers inside an XCD in the LDS-tile bodies: the control wave and
// worker waves 4..6 (which have no weight copy in flight).
constexpr int kPollWaves = 4;

// A worker wave's share (part 1..NP-1) of a gather the control wave publishes into;
// false if the wait gave up.
template <int KP, int NP = kPollWaves>
__device__ __forceinline__ bool help_gather(const u64* src, int n, uint32_t tag, float* dst, int own0, int own1, int part,
                                            int lane, const Params& P) {
  uint32_t rounds = 0;
  unsigned long long r1 = 0;
  return exchange<KP, NP>(src, n, tag, dst, own0, own1, [] {}, lane, P, rounds, r1, part);
}
// The attention-chunk gather is polled by all eight waves (the control wave part 0, worker
// wave w part w + 1): in the LDS-tile bodies the copy waves issue that segment's copies
// after their part; in the register-tile body the ring heads in flight then were issued
// an exchange and the attention earlier.  Long contexts gather 32 chunks there.
template <class B>
constexpr int comb_parts() { return kWorkerWaves + 1; }

// Phase trace: one workgroup (dbg_phase_wg >= 0, records [n][n_sync][8]) or every
// workgroup (dbg_phase_wg < 0, records [n][grid][n_sync][8]).
__device__ __forceinline__ bool phase_traced(const Params& P, int b) {
  return P.dbg_phase != nullptr && (P.dbg_phase_wg < 0 || b == P.dbg_phase_wg);
}
__device__ __forceinline__ unsigned long long* phase_record(const Params& P, int b, int t, int n_sync, int ph) {
  const size_t per_t = (size_t)n_sync * (P.dbg_phase_wg < 0 ? kGrid : 1);
  const size_t wg = P.dbg_phase_wg < 0 ? (size_t)b : 0;
  return P.dbg_phase + ((size_t)t * per_t + wg * n_sync + ph) * 8;
}

// ------------------------------------------------------------------ GEMV tiles
// Issue the wave's loads of a tile.  Unconditional on purpose: waves without rows
// and chunks past the tile read the last valid chunk (never used), so the compiler
// never has to merge loaded and unloaded register states.
template <class T>
__device__ __forceinline__ void tile_load(T& t, const uint8_t* base, int wave, int lane) {
  const int w = min(wave, T::NWA - 1);
  const u4* p = reinterpret_cast<const u4*>(base);
#pragma unroll
  for (int j = 0; j < T::LPL; ++j) {
    const int g = w * T::CPW + j * 64 + lane;
    t.v[j] = __builtin_nontemporal_load(p + (T::EXACT ? g : min(g, T::TOTAL - 1)));
  }
}

template <class B>
__device__ __forceinline__ float dot_chunk(const u4& w, const float* a) {
  if constexpr (B::BF16) {
    const f4 a0 = *reinterpret_cast<const f4*>(a);
    const f4 a1 = *reinterpret_cast<const f4*>(a + 4);
    float s = bf16lo(w.x) * a0.x;
    s = fmaf(bf16hi(w.x), a0.y, s);
    s = fmaf(bf16lo(w.y), a0.z, s);
    s = fmaf(bf16hi(w.y), a0.w, s);
    s = fmaf(bf16lo(w.z), a1.x, s);
    s = fmaf(bf16hi(w.z), a1.y, s);
    s = fmaf(bf16lo(w.w), a1.z, s);
    s = fmaf(bf16hi(w.w), a1.w, s);
    return s;
  } else {
    const f4 a0 = *reinterpret_cast<const f4*>(a);
    float s = __uint_as_float(w.x) * a0.x;
    s = fmaf(__uint_as_float(w.y), a0.y, s);
    s = fmaf(__uint_as_float(w.z), a0.z, s);
    s = fmaf(__uint_as_float(w.w), a0.w, s);
    return s;
  }
}

// Row results of the wave's rows go to res[wave*RPW + r] (LDS).
template <class B, class T>
__device__ __forceinline__ void tile_dot(const T& t, const float* act, float* res, int wave, int lane) {
  if (wave >= T::NWA) return;
  float acc[T::RPW];
#pragma unroll
  for (int r = 0; r < T::RPW; ++r) acc[r] = 0.f;
#pragma unroll
  for (int j = 0; j < T::LPL; ++j) {
    const int k = j * 64 + lane;
    if (T::EXACT || (k < T::CPW && wave * T::CPW + k < T::TOTAL)) {
      const int row = k / T::CPR;
      const int col = (k - row * T::CPR) * B::E;
      const float d = dot_chunk<B>(t.v[j], act + col);
      if constexpr (T::CPR % 64 == 0) {
        acc[(j * 64) / T::CPR] += d;
      } else {
#pragma unroll
        for (int r = 0; r < T::RPW; ++r) acc[r] += (row == r) ? d : 0.f;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < T::RPW; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < T::RPW; ++r)
      if (wave * T::RPW + r < T::TOTAL / T::CPR)
        res[wave * T::RPW + r] = acc[r];
  }
}

// A tile streamed from HBM through a ring of kRing chunks per lane: the first kRing
// 1 KB loads of the wave's rows are issued ahead (stream_begin, one exchange before the
// dot product), and the dot product issues load j + kRing as it consumes chunk j, so a
// wave keeps kRing KB in flight instead of holding its whole share of the tile.  The
// loads are buffer loads over the wave's rows (one lane offset, the chunk in the
// constant offset, so no address registers per chunk; past the tile they read 0).
constexpr int kRing = 8;
constexpr int kNonTemporal = 2;  // cache-policy bit of a buffer load: streamed
struct Ring {
  u4 v[kRing];
  __amdgpu_buffer_rsrc_t src;
  int last;  // byte offset of the wave's last 1 KB instruction: later chunks re-read it
};
// Chunk j of the wave's rows (instructions past its rows re-read its last one: every load
// stays inside the tile, and the dot product ignores them).
template <class T>
__device__ __forceinline__ u4 stream_load(const Ring& q, int j, int lane) {
  return __builtin_amdgcn_raw_buffer_load_b128(q.src, lane * 16, min(j * 1024, q.last), kNonTemporal);
}
template <class T>
__device__ __forceinline__ void stream_begin(Ring& q, const uint8_t* base, int wave, int lane) {
  static_assert(T::CPW % 64 == 0 && T::TOTAL % 64 == 0 && T::TOTAL >= 64, "whole 1 KB instructions");
  // the wave's rows; a wave past the last row reads the tile's last instruction (ignored)
  const int start = min(min(wave, T::NWA - 1) * T::CPW, T::TOTAL - 64);
  const int chunks = min(T::CPW, T::TOTAL - start);
  q.src = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base) + (size_t)start * 16, (short)0, chunks * 16,
                                            0x00020000);
  q.last = (chunks / 64 - 1) * 1024;
#pragma unroll
  for (int j = 0; j < kRing; ++j)
    if (j < T::LPL) q.v[j] = stream_load<T>(q, j, lane);
}
// Row results of the wave's rows go to res[wave*RPW + r] (LDS), as tile_dot.
template <class B, class T>
__device__ __forceinline__ void stream_dot(Ring& q, const float* act, float* res, int wave, int lane) {
  if (wave >= T::NWA) return;  // (its ring loads are in bounds and simply not used)
  float acc[T::RPW];
#pragma unroll
  for (int r = 0; r < T::RPW; ++r) acc[r] = 0.f;
#pragma unroll
  for (int j = 0; j < T::LPL; ++j) {
    const u4 w = q.v[j % kRing];
    if (j + kRing < T::LPL) q.v[j % kRing] = stream_load<T>(q, j + kRing, lane);
    const int k = j * 64 + lane;
    if (T::EXACT || (k < T::CPW && wave * T::CPW + k < T::TOTAL)) {
      const int row = k / T::CPR;
      const int col = (k - row * T::CPR) * B::E;
      const float d = dot_chunk<B>(w, act + col);
      if constexpr (T::CPR % 64 == 0) {
        acc[(j * 64) / T::CPR] += d;
      } else {
        // the 64 chunks of load j span rows r0 and at most r0 + 1; once the loops are
        // unrolled r0 is a constant and only those two accumulators are touched
        static_assert(T::CPR >= 64 || (64 % T::CPR == 0 && T::CPR >= 32), "two rows per load at most");
        const int r0 = (j * 64) / T::CPR;
        const bool next = row > r0;
#pragma unroll
        for (int r = 0; r < T::RPW; ++r) {
          if (r == r0) acc[r] += next ? 0.f : d;
          else if (r == r0 + 1) acc[r] += next ? d : 0.f;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < T::RPW; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < T::RPW; ++r)
      if (wave * T::RPW + r < T::TOTAL / T::CPR)
        res[wave * T::RPW + r] = acc[r];
  }
}

// tile_dot with the tile in LDS: chunk g of the tile at slot[g].
template <class B, class T>
__device__ __forceinline__ void tile_dot_lds(const u4* slot, const float* act, float* res, int wave, int lane) {
  if (wave >= T::NWA) return;
  float acc[T::RPW];
#pragma unroll
  for (int r = 0; r < T::RPW; ++r) acc[r] = 0.f;
#pragma unroll
  for (int j = 0; j < T::LPL; ++j) {
    const int k = j * 64 + lane;
    if (T::EXACT || (k < T::CPW && wave * T::CPW + k < T::TOTAL)) {
      const u4 w = slot[wave * T::CPW + k];
      const int row = k / T::CPR;
      const int col = (k - row * T::CPR) * B::E;
      const float d = dot_chunk<B>(w, act + col);
      if constexpr (T::CPR % 64 == 0) {
        acc[(j * 64) / T::CPR] += d;
      } else {
#pragma unroll
        for (int r = 0; r < T::RPW; ++r) acc[r] += (row == r) ? d : 0.f;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < T::RPW; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < T::RPW; ++r)
      if (wave * T::RPW + r < T::TOTAL / T::CPR) res[wave * T::RPW + r] = acc[r];
  }
}



// A GEMV tile of ROWS rows x COLS bf16 weights in LDS (chunk g at slot[g], row-major).
// Worker wave w takes rows [w*RPW, w*RPW + RPW); the row loop has a fixed trip count and
// no branches (rows past the tile re-read the last row and are not stored), so the rows'
// loads, products and reductions interleave.  A row of CPR < 64 chunks (CPR dividing 64)
// is one group of CPR lanes, 64/CPR rows per pass; a longer row takes ceil(CPR/64) passes
// over the wave's lanes.
template <int ROWS, int COLS>
struct Gemv2 {
  static constexpr int CPR = COLS / 8;
  // the seven worker waves and the control wave (waves w and w + 4 share a SIMD, so equal
  // shares over all eight balance the SIMDs)
  static constexpr int RPW = (ROWS + kWorkerWaves) / (kWorkerWaves + 1);
  static constexpr bool GROUPED = CPR < 64 && 64 % CPR == 0;
  static constexpr int RPI = GROUPED ? 64 / CPR : 1;  // rows per pass
  static constexpr int NPASS = (RPW + RPI - 1) / RPI;
  static constexpr int NIT = GROUPED ? 1 : (CPR + 63) / 64;
  static_assert(COLS % 8 == 0 && ROWS <= 64, "tile");
};

// 8 fp32 inputs of chunk c as hi/lo bf16 chunks, times the gains g when GAIN.
template <bool GAIN>
__device__ __forceinline__ void split_chunk(const f4 (&v)[2], const float* g, int c, u4& hi, u4& lo) {
  float y[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
  if constexpr (GAIN) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f4 gg = *reinterpret_cast<const f4*>(g + 8 * c + 4 * e);
      y[4 * e + 0] *= gg.x;
      y[4 * e + 1] *= gg.y;
      y[4 * e + 2] *= gg.z;
      y[4 * e + 3] *= gg.w;
    }
  }
  split8(y, hi, lo);
}

// Input of a bf16 GEMV with LDS tiles: fp32 in LDS (each wave splits the chunks it reads),
// fp32 RMS-normalised on the way, or already split into hi/lo chunks in LDS.
enum class In { kF32, kF32Norm, kSplit };

// Rows [wave*RPW, ...) of a ROWS x COLS bf16 tile in LDS times the input x, into res.  For
// In::kSplit, x points at the hi chunks and g at the lo chunks.  Every wave splits the
// fp32 input chunks it reads itself.  With In::kF32Norm the input is
// RMS-normalised with gains g: the products run on g * x, and each row sum is scaled by
// 1/rms(x) at the end (one scalar per input vector), so the wave's sum of squares over all
// COLS inputs overlaps the products instead of preceding them.  Every wave sums in the
// same order (lane L's chunks are L, L + 64, ...), so all waves use the same scale.
template <int ROWS, int COLS, In IN>
__device__ __forceinline__ void tile_dot2(const u4* slot, const float* x, const float* g, float eps, float* res, int wave,
                                          int lane) {
  constexpr bool NORM = IN == In::kF32Norm;
  using G = Gemv2<ROWS, COLS>;
  constexpr int CPR = G::CPR;
  const int r0 = wave * G::RPW;
  if (r0 >= ROWS) return;
  if constexpr (G::GROUPED) {
    static_assert(!NORM, "normalised inputs use the chunk-per-lane layout");
    const int lr = lane / CPR, c = lane % CPR;
    u4 hi, lo;
    if constexpr (IN == In::kSplit) {
      hi = reinterpret_cast<const u4*>(x)[c];
      lo = reinterpret_cast<const u4*>(g)[c];
    } else {
      f4 v[2];
      v[0] = *reinterpret_cast<const f4*>(x + 8 * c);
      v[1] = *reinterpret_cast<const f4*>(x + 8 * c + 4);
      split_chunk<false>(v, g, c, hi, lo);
    }
    float d[G::NPASS];
#pragma unroll
    for (int i = 0; i < G::NPASS; ++i) {
      const int row = min(r0 + i * G::RPI + lr, ROWS - 1);
      d[i] = dot8(slot[row * CPR + c], hi, lo, 0.f);
    }
#pragma unroll
    for (int i = 0; i < G::NPASS; ++i) d[i] = group_sum<CPR>(d[i]);
#pragma unroll
    for (int i = 0; i < G::NPASS; ++i) {
      const int j = i * G::RPI + lr, row = r0 + j;
      if (c == CPR - 1 && j < G::RPW && row < ROWS) res[row] = d[i];
    }
  } else {
    f4 v[G::NIT][2];
    u4 hi[G::NIT], lo[G::NIT];
#pragma unroll
    for (int i = 0; i < G::NIT; ++i) {
      const int c = min(lane + 64 * i, CPR - 1);
      if constexpr (IN == In::kSplit) {
        hi[i] = reinterpret_cast<const u4*>(x)[c];
        lo[i] = reinterpret_cast<const u4*>(g)[c];
      } else {
        v[i][0] = *reinterpret_cast<const f4*>(x + 8 * c);
        v[i][1] = *reinterpret_cast<const f4*>(x + 8 * c + 4);
        split_chunk<NORM>(v[i], g, c, hi[i], lo[i]);
      }
    }
    float rs = 1.f;
    if constexpr (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < G::NIT; ++i) {
        if (CPR % 64 == 0 || lane + 64 * i < CPR) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            ss = fmaf(v[i][e].x, v[i][e].x, ss);
            ss = fmaf(v[i][e].y, v[i][e].y, ss);
            ss = fmaf(v[i][e].z, v[i][e].z, ss);
            ss = fmaf(v[i][e].w, v[i][e].w, ss);
          }
        }
      }
      ss = wave_sum(ss);
      rs = __builtin_amdgcn_rsqf(ss / (float)COLS + eps);
    }
    float d[G::RPW];
#pragma unroll
    for (int j = 0; j < G::RPW; ++j) {
      const int row = min(r0 + j, ROWS - 1);
      d[j] = 0.f;
#pragma unroll
      for (int i = 0; i < G::NIT; ++i) {
        const int c = lane + 64 * i;
        const u4 w = slot[row * CPR + min(c, CPR - 1)];
        if (CPR % 64 == 0 || c < CPR) d[j] = dot8(w, hi[i], lo[i], d[j]);
      }
    }
    // the wave's row sums together: lane L ends with row L / (64 / NS)
    constexpr int NS = G::RPW <= 2 ? 2 : (G::RPW <= 4 ? 4 : (G::RPW <= 8 ? 8 : 16));
    static_assert(G::RPW <= 16, "rows per wave");
    float dv[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) dv[j] = j < G::RPW ? d[j] : 0.f;
    const float tot = transpose_sum<NS>(dv, lane);
    constexpr int GL = 64 / NS;
    const int j = lane / GL;
    if (lane % GL == GL - 1 && j < G::RPW && r0 + j < ROWS) res[r0 + j] = NORM ? tot * rs : tot;
  }
}

// ------------------------------------------------------------------ the kernel
template <class B>
struct Lds {
  alignas(16) float xs[B::H];            // residual stream (every workgroup holds all of it)
  alignas(16) float an[B::H];            // normalised input of the next GEMV
  alignas(16) float qkv[B::RQKV];        // raw q,k,v of this XCD's group, then q rotated and scaled
  float kp[B::D], vp[B::D];  // K and V of the current position (cache precision)
  alignas(16) float ov[B::OC];           // attention output of the group
  alignas(16) float mv[B::IX];           // SwiGLU output slice
  alignas(16) float res[64];             // row results of the current tile
  u4 ov_hi[B::OC / 8], ov_lo[B::OC / 8];  // attention output split for the O GEMV (bf16 hi, lo)
  alignas(16) float part[kPerXcd][B::QPG][B::D + 2];        // chunk partials read back for the combine
  alignas(16) float wpart[kWorkerWaves][B::QPG][B::D + 2];  // per-wave attention partials
  alignas(16) float attw[kWorkerWaves][16];                 // per-wave softmax weights of a batch
  alignas(16) float chw[kWorkerWaves + 1][64];              // per-wave chunk weights of the combine
  float wbest_v[kWorkerWaves];
  int wbest_i[kWorkerWaves];
  alignas(16) float g_in0[B::H];         // input norm of layer 0 (constant for the launch)
  // gains of layer j in G[j % 2] (j counted from the launch start), filled by the workers
  // ahead of use: [post-attention norm H][q norm D][k norm D][input norm of the next layer H],
  // each buffer padded to whole KB because an LDS copy instruction always writes 1 KB
  alignas(16) float G[2][(2 * B::H + 2 * B::D + 255) / 256 * 256];
  float rope_c[B::D / 2], rope_s[B::D / 2];  // cos/sin of every rotary pair at this position
  int abort_;
};


// Attention at position p covers positions 0..p, cut into n_chunks contiguous chunks
// of chunk_len positions; chunk r goes to rank r of the group's XCD.  At most 28 chunks
// in the LDS-tile bodies and 24 in the H = 2048 body (measured: fewer, longer chunks
// shorten the combine's gather more than they lengthen the attention at long contexts).
constexpr int kMinChunk = 56;  // one batch of 8 positions per worker wave
template <class B>
constexpr int kMaxChunks = B::H <= 1024 ? 28 : 24;
template <class B>
__device__ __forceinline__ int n_chunks(int p) {
  return min(kMaxChunks<B>, max(1, (p + 1 + kMinChunk - 1) / kMinChunk));
}

// RMSNorm of x with gains g into out (fp32), lane L working on 8-element chunks L,
// L + 64, ... (16-byte LDS accesses; the order of the sum of squares is the one the bf16
// GEMVs that normalise their own inputs use).
template <class B>
__device__ __forceinline__ void norm_out(const float* x, const float* g, float* out, float eps, int lane) {
  constexpr int NCH = B::H / 8, CPL = (NCH + 63) / 64;
  f4 v[CPL][2];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = min(lane + 64 * i, NCH - 1);
    v[i][0] = *reinterpret_cast<const f4*>(x + 8 * c);
    v[i][1] = *reinterpret_cast<const f4*>(x + 8 * c + 4);
    if (NCH % 64 == 0 || lane + 64 * i < NCH) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        ss = fmaf(v[i][e].x, v[i][e].x, ss);
        ss = fmaf(v[i][e].y, v[i][e].y, ss);
        ss = fmaf(v[i][e].z, v[i][e].z, ss);
        ss = fmaf(v[i][e].w, v[i][e].w, ss);
      }
    }
  }
  ss = wave_sum(ss);
  const float rs = __builtin_amdgcn_rsqf(ss / (float)B::H + eps);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (NCH % 64 == 0 || c < NCH) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const f4 gg = *reinterpret_cast<const f4*>(g + 8 * c + 4 * e);
        *reinterpret_cast<f4*>(out + 8 * c + 4 * e) =
            f4{gg.x * (v[i][e].x * rs), gg.y * (v[i][e].y * rs), gg.z * (v[i][e].z * rs), gg.w * (v[i][e].w * rs)};
      }
    }
  }
}

template <class B>
__device__ __forceinline__ void norm_to(const float* x, const float* g, float* out, float eps, int lane) {
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < B::HPL; ++k) { const float v = x[lane + 64 * k]; ss = fmaf(v, v, ss); }
  ss = wave_sum(ss);
  const float rs = __builtin_amdgcn_rsqf(ss / (float)B::H + eps);
#pragma unroll
  for (int k = 0; k < B::HPL; ++k) { const int i = lane + 64 * k; out[i] = g[i] * (x[i] * rs); }
}

// ---------------------------------------------------------------- shared steps after a gather
// With the tiles in LDS, all eight waves of a workgroup take part in the steps that follow
// the q/k/v gather and the attention gather, wave pw doing share pw of 8 (the control
// wave is pw 7).

// Per-head RMSNorm of q and k and their rotation (head dim 128: lane i holds elements i and
// i + 64 of a head, rotary pair i), the cache rounding of k and v: q head pw (pw < QPG),
// k (pw == QPG), v (pw == QPG + 1).
template <class B>
__device__ __forceinline__ void qk_part(Lds<B>& S, const float* qn, const float* kn, float eps, bool kv_bf16, int pw,
                                        int lane) {
  static_assert(B::D == 128, "two elements per lane");
  if (pw <= B::QPG) {
    const float a0 = S.qkv[pw * B::D + lane], a1 = S.qkv[pw * B::D + lane + 64];
    const float ss = wave_sum(fmaf(a1, a1, a0 * a0));
    const float* g = pw < B::QPG ? qn : kn;
    const float rs = __builtin_amdgcn_rsqf(ss / (float)B::D + eps);
    const float c = S.rope_c[lane], sn = S.rope_s[lane];
    const float n0 = g[lane] * (a0 * rs), n1 = g[lane + 64] * (a1 * rs);
    float o0 = n0 * c - n1 * sn, o1 = n1 * c + n0 * sn;
    if (pw < B::QPG) {
      const float qscale = rsqrtf((float)B::D);
      S.qkv[pw * B::D + lane] = o0 * qscale;
      S.qkv[pw * B::D + lane + 64] = o1 * qscale;
    } else {
      if (kv_bf16) { o0 = bf16_round(o0); o1 = bf16_round(o1); }
      S.kp[lane] = o0;
      S.kp[lane + 64] = o1;
    }
  } else if (pw == B::QPG + 1) {
    const float v0 = S.qkv[(B::QPG + 1) * B::D + lane], v1 = S.qkv[(B::QPG + 1) * B::D + lane + 64];
    S.vp[lane] = kv_bf16 ? bf16_round(v0) : v0;
    S.vp[lane + 64] = kv_bf16 ? bf16_round(v1) : v1;
  }
}

// RMSNorm of x with gains g into out (fp32), wave pw writing chunks [pw*H/64, ...): every
// wave sums the squares of all of x in norm_out's order, so all use one scale.
template <class B>
__device__ __forceinline__ void norm_out_part(const float* x, const float* g, float* out, float eps, int pw, int lane) {
  constexpr int NCH = B::H / 8, CPL = NCH / 64, CPW = NCH / 8;
  static_assert(NCH % 64 == 0 && CPW <= 64, "whole chunks per lane and per wave");
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f4 v = *reinterpret_cast<const f4*>(x + 8 * c + 4 * e);
      ss = fmaf(v.x, v.x, ss);
      ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss);
      ss = fmaf(v.w, v.w, ss);
    }
  }
  ss = wave_sum(ss);
  const float rs = __builtin_amdgcn_rsqf(ss / (float)B::H + eps);
  if (lane < CPW) {
    const int c = pw * CPW + lane;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f4 v = *reinterpret_cast<const f4*>(x + 8 * c + 4 * e);
      const f4 gg = *reinterpret_cast<const f4*>(g + 8 * c + 4 * e);
      *reinterpret_cast<f4*>(out + 8 * c + 4 * e) = f4{gg.x * (v.x * rs), gg.y * (v.y * rs), gg.z * (v.z * rs), gg.w * (v.w * rs)};
    }
  }
}

// The group's attention output from the nc chunk partials in S.part, split for the O
// GEMV: wave pw takes output columns [pw*QPG*D/8, ...) of one head.  Lane c first works
// out chunk c's weight exp(m_c - M) (M the largest chunk maximum) and the weights go
// through LDS; then lane = column sums the chunks' vectors in chunk order, and four lanes
// split the wave's columns 8 at a time.
template <class B>
__device__ __forceinline__ void combine_part(Lds<B>& S, int nc, int pw, int lane) {
  constexpr int CW = B::OC / 8;  // columns per wave
  static_assert(CW <= 64 && CW % 8 == 0 && B::D % CW == 0 && kPerXcd <= 64, "columns per wave, a chunk per lane");
  const int col = pw * CW + lane, h = (pw * CW) / B::D, d = col - h * B::D;
  const int cl = min(lane, nc - 1);
  const float mc = lane < nc ? S.part[cl][h][0] : -INFINITY;
  const float M = wave_max(mc);
  const float f = (lane < nc && mc != -INFINITY) ? __expf(mc - M) : 0.f;
  const float Ls = wave_sum(S.part[cl][h][1] * f);
  S.chw[pw][lane] = f;  // this wave's own LDS writes are seen by its later reads
  if (lane < CW) {
    // the weights past nc are zero and the chunk index is clamped, so the loop may run
    // past nc: in the LDS-tile bodies it is unrolled to the next of 8, 16 or 32 chunks
    // (all LDS reads independent); the H = 2048 body keeps a loop (its registers are full)
    auto sum_chunks = [&](auto n_max) {
      constexpr int NM = decltype(n_max)::value;
      float a = 0.f;
#pragma unroll
      for (int c0 = 0; c0 < NM; c0 += 4) {
        const f4 w = *reinterpret_cast<const f4*>(&S.chw[pw][c0]);  // zero past nc
        a = fmaf(S.part[min(c0 + 0, nc - 1)][h][2 + d], w.x, a);
        a = fmaf(S.part[min(c0 + 1, nc - 1)][h][2 + d], w.y, a);
        a = fmaf(S.part[min(c0 + 2, nc - 1)][h][2 + d], w.z, a);
        a = fmaf(S.part[min(c0 + 3, nc - 1)][h][2 + d], w.w, a);
      }
      return a;
    };
    float a = 0.f;
    if constexpr (B::H <= 1024) {
      a = nc <= 8    ? sum_chunks(std::integral_constant<int, 8>{})
          : nc <= 16 ? sum_chunks(std::integral_constant<int, 16>{})
                     : sum_chunks(std::integral_constant<int, kPerXcd>{});
    } else {
      for (int c0 = 0; c0 < nc; c0 += 4) {
        const f4 w = *reinterpret_cast<const f4*>(&S.chw[pw][c0]);  // zero past nc
        a = fmaf(S.part[min(c0 + 0, nc - 1)][h][2 + d], w.x, a);
        a = fmaf(S.part[min(c0 + 1, nc - 1)][h][2 + d], w.y, a);
        a = fmaf(S.part[min(c0 + 2, nc - 1)][h][2 + d], w.z, a);
        a = fmaf(S.part[min(c0 + 3, nc - 1)][h][2 + d], w.w, a);
      }
    }
    S.ov[col] = a * __builtin_amdgcn_rcpf(Ls);
  }
  if (lane < CW / 8) split8(S.ov + pw * CW + 8 * lane, S.ov_hi[pw * (CW / 8) + lane], S.ov_lo[pw * (CW / 8) + lane]);
}

// Addresses of this workgroup's tiles in layer l.
template <class B>
struct TileAddr {
  const Params& P;
  int x, r;
  __device__ const uint8_t* layer(int l) const { return P.layers + (size_t)l * P.lay.stride; }
  // XCDs without a KV group (fewer groups than XCDs) address group x % NG: in bounds, unused
  __device__ const uint8_t* qkv(int l) const {
    return layer(l) + P.lay.qkv + ((size_t)(x % B::NG) * B::RQKV + (size_t)r * B::T_QKV) * B::H * B::WB;
  }
  __device__ const uint8_t* o(int l) const {
    return layer(l) + P.lay.o + ((size_t)(x % B::NG) * B::H + (size_t)r * B::T_O) * B::OC * B::WB;
  }
  __device__ const uint8_t* gu(int l) const {
    return layer(l) + P.lay.gu + ((size_t)x * kPerXcd + r) * (size_t)B::T_GU * B::H * B::WB;
  }
  __device__ const uint8_t* down(int l) const {
    return layer(l) + P.lay.down + ((size_t)x * B::H + (size_t)r * B::T_D) * B::IX * B::WB;
  }
  __device__ const uint8_t* gains(int l) const { return layer(l) + P.lay.gains; }
};

// Bodies whose QKV and gate/up tiles fit in one LDS slot and O and down tiles in another
// stream their tiles through LDS; the larger body holds them in registers, one phase ahead.
template <class B>
constexpr bool lds_tiles() { return B::H <= 1024; }
template <class B>
constexpr int slot_a_bytes() { return lds_tiles<B>() ? (int)((((B::T_QKV > B::T_GU ? B::T_QKV : B::T_GU) * B::H * B::WB + 1023) / 1024) * 1024) : 16; }
template <class B>
constexpr int slot_b_bytes() {
  return lds_tiles<B>() ? (int)((((B::T_O * B::OC > B::T_D * B::IX ? B::T_O * B::OC : B::T_D * B::IX) * B::WB + 1023) / 1024) * 1024) : 16;
}
constexpr int kGainFloats(int H, int D) { return 2 * H + 2 * D; }

// copy in flight, so they can take part in the gathers of other workgroups' words (a wave's
// vector-memory counter is in order: a poll could not complete before an earlier copy).
constexpr int kDmaWaves = 4;
// Copy `chunks` 16-byte chunks src -> lds; instruction i (64 chunks) is issued by wave i % 4.
template <int CHUNKS>
__device__ __forceinline__ void dma_copy(const uint8_t* src, void* lds, int wave, int lane) {
  constexpr int NI = (CHUNKS + 63) / 64;
  if (wave >= kDmaWaves) return;
  for (int i = wave; i < NI; i += kDmaWaves) {
    const int g = min(i * 64 + lane, CHUNKS - 1);
    lds_dma16(src + (size_t)g * 16, reinterpret_cast<uint8_t*>(lds) + (size_t)i * 1024);
  }
}
// Part `part` of NPARTS of the same copy: its 1 KB instructions [part*NI/NPARTS,
// (part+1)*NI/NPARTS), instruction i issued by wave i % 4 as in the whole copy.
template <int CHUNKS, int NPARTS>
__device__ __forceinline__ void dma_part(const uint8_t* src, void* lds, int part, int wave, int lane) {
  constexpr int NI = (CHUNKS + 63) / 64;
  if (wave >= kDmaWaves) return;
  const int a = part * NI / NPARTS, b = (part + 1) * NI / NPARTS;
  for (int i = a + (wave - a % kDmaWaves + kDmaWaves) % kDmaWaves; i < b; i += kDmaWaves) {
    const int g = min(i * 64 + lane, CHUNKS - 1);
    lds_dma16(src + (size_t)g * 16, reinterpret_cast<uint8_t*>(lds) + (size_t)i * 1024);
  }
}

// ------------------------------------------------------------------ worker waves
// LM head rows of one pass: 2 per worker wave from rb, wave w holds rows rb + 2w, rb + 2w + 1.
// Rows at or past row_end read row_end-1 (in bounds, ignored by the argmax).
template <class B, class T>
__device__ __forceinline__ void lm_load(T& tl, const Params& P, int rb, int row_end, int wave, int lane) {
  const int last = max(0, row_end - 1);
#pragma unroll
  for (int j = 0; j < T::LPL; ++j) {
    const int k = min(j * 64 + lane, T::CPW - 1);
    const int row = min(rb + wave * T::RPW + k / T::CPR, last);
    const u4* p = reinterpret_cast<const u4*>(reinterpret_cast<const uint8_t*>(P.lm_head) + (size_t)row * B::H * B::WB);
    tl.v[j] = __builtin_nontemporal_load(p + (k - (k / T::CPR) * T::CPR));
  }
}

template <class B, class T>
__device__ __forceinline__ void lm_dot(const T& tl, const float* an, int rb, int row_end, int wave, int lane,
                                       float& bv, int& bi) {
  float acc[T::RPW];
#pragma unroll
  for (int q = 0; q < T::RPW; ++q) acc[q] = 0.f;
#pragma unroll
  for (int j = 0; j < T::LPL; ++j) {
    const int k = j * 64 + lane;
    if (T::CPW % 64 == 0 || k < T::CPW) {
      const int row = k / T::CPR;
      const float d = dot_chunk<B>(tl.v[j], an + (k - row * T::CPR) * B::E);
#pragma unroll
      for (int q = 0; q < T::RPW; ++q) acc[q] += (row == q) ? d : 0.f;
    }
  }
#pragma unroll
  for (int q = 0; q < T::RPW; ++q) {
    const float v = wave_sum(acc[q]);
    const int row = rb + wave * T::RPW + q;
    if (row < row_end && (v > bv || (v == bv && row < bi))) { bv = v; bi = row; }
  }
}

// Attention of this rank's chunk [c0, c1) of positions for the group's query heads.  A
// cache row (one position's K or V of one KV head) is 256 bytes: 16 lanes hold 16 bytes
// each, so one load instruction covers 4 positions (lane group sub = lane / 16).  Each
// worker wave takes a contiguous share of the chunk; all its row loads of a batch are in
// flight together (device-coherent 128-bit buffer loads).  Every lane group keeps an online
// softmax over its positions; the four groups are merged at the end.  The current position
// p is taken from LDS (K rotated and both rounded to cache precision by the control wave).
// The KV cache entry of group x at position p (layer l), from the rotated and rounded
// k and v of this step in LDS.  Written by one worker wave of the group's last rank,
// which waits for the stores to complete before it arrives at the next barrier: the
// entry is visible to every reader of a later step.
template <class B>
__device__ __forceinline__ void write_kv_entry(const Params& P, const Lds<B>& S, int x, int l, int p, int lane) {
  const size_t off = (((size_t)l * B::NKV + x) * P.max_seq + p) * B::D;
#pragma unroll
  for (int k = 0; k < B::DPL; ++k) {
    const int i = lane + 64 * k;
    if (P.kv_bf16) {
      __hip_atomic_store(reinterpret_cast<uint16_t*>(P.kcache) + off + i, f_to_bf16(S.kp[i]), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(reinterpret_cast<uint16_t*>(P.vcache) + off + i, f_to_bf16(S.vp[i]), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    } else {
      __hip_atomic_store(reinterpret_cast<float*>(P.kcache) + off + i, S.kp[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(reinterpret_cast<float*>(P.vcache) + off + i, S.vp[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // every store of this wave acknowledged (and every copy landed)
}

// Attention over cache positions [c0, c1) of KV group x at layer l, for the group's
// query heads.  A wave reads whole cache rows: lane i holds head dims
// [i*DPL, i*DPL + DPL) of every row (one 4-byte load per lane and row), so a position's
// score is one wave sum, uniform across the wave, and the wave's positions need no merge.
// Position p comes from LDS (k/v of this step).  The positions of a wave are taken
// kAttnBatch at a time, online softmax across batches.
constexpr int kAttnBatch = 8;
constexpr int kCoherent = 16;  // cache-policy bit of a buffer load: device-coherent

template <class B>
struct KvBatch {
  uint32_t k[kAttnBatch], v[kAttnBatch];
};

template <class B>
struct KvRange {
  __amdgpu_buffer_rsrc_t rk, rv;
  int w0, w1;  // this wave's positions
};

template <class B>
__device__ __forceinline__ KvRange<B> kv_range(const Params& P, int x, int l, int c0, int c1, int wave) {
  constexpr int ROWB = B::D * (B::BF16 ? 2 : 4);
  const int n = c1 - c0;
  const int per = (n + kWorkerWaves - 1) / kWorkerWaves;
  KvRange<B> R;
  R.w0 = c0 + wave * per;
  R.w1 = min(c1, R.w0 + per);
  const size_t row0 = ((size_t)l * B::NKV + x) * P.max_seq;
  const int nbytes = P.max_seq * ROWB;
  R.rk = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<uint8_t*>(P.kcache) + row0 * ROWB, (short)0, nbytes, 0x00020000);
  R.rv = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<uint8_t*>(P.vcache) + row0 * ROWB, (short)0, nbytes, 0x00020000);
  return R;
}

// Issue the loads of one batch: positions jb + u, clamped into the range (rows past it are
// loaded again and ignored).  The row of the current position may hold data of an earlier
// call: the caller takes that position from LDS.
template <class B>
__device__ __forceinline__ void kv_batch_load(const KvRange<B>& R, int jb, int lane, KvBatch<B>& kb) {
  constexpr int ROWB = B::D * (B::BF16 ? 2 : 4);
  static_assert(ROWB == 256, "a cache row is 64 lanes x 4 bytes");
#pragma unroll
  for (int u = 0; u < kAttnBatch; ++u) {
    const int jj = max(min(jb + u, R.w1 - 1), 0);
    kb.k[u] = __builtin_amdgcn_raw_buffer_load_b32(R.rk, jj * ROWB + lane * 4, 0, kCoherent);
    kb.v[u] = __builtin_amdgcn_raw_buffer_load_b32(R.rv, jj * ROWB + lane * 4, 0, kCoherent);
  }
}

// The first batch of a wave's positions, loaded ahead of the attention phase: the cache
// rows before position p do not depend on this step, so they can be in flight while
// the q/k/v rows are computed and exchanged.
template <class B>
__device__ __forceinline__ void attention_prefetch(const Params& P, int x, int l, int c0, int c1, int wave, int lane,
                                                   KvBatch<B>& kb) {
  const KvRange<B> R = kv_range<B>(P, x, l, c0, c1, wave);
  if (R.w0 < R.w1) kv_batch_load<B>(R, R.w0, lane, kb);
}

template <class B, bool PREFETCHED>
__device__ __forceinline__ void attention_chunk(const Params& P, Lds<B>& S, int x, int l, int p, int c0, int c1,
                                                int wave, int lane, const KvBatch<B>& first) {
  constexpr int DPL = B::D / 64;  // head dims per lane: 2 (bf16, d = 128) or 1 (f32, d = 64)
  static_assert(DPL * (B::BF16 ? 2 : 4) == 4, "one 4-byte word per lane and row");
  constexpr int PB = kAttnBatch;
  float q[B::QPG][DPL];
#pragma unroll
  for (int h = 0; h < B::QPG; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) q[h][e] = S.qkv[h * B::D + lane * DPL + e];
  float m[B::QPG], ls[B::QPG], acc[B::QPG][DPL];
#pragma unroll
  for (int h = 0; h < B::QPG; ++h) {
    m[h] = -INFINITY;
    ls[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
  }
  auto widen = [&](uint32_t w, float (&f)[DPL]) {
    if constexpr (B::BF16) {
      f[0] = bf16lo(w);
      f[1] = bf16hi(w);
    } else {
      f[0] = __uint_as_float(w);
    }
  };
  const KvRange<B> R = kv_range<B>(P, x, l, c0, c1, wave);
  const int w0 = R.w0, w1 = R.w1;
  auto batch = [&](const KvBatch<B>& kb, int jb) {
    const int nb = min(PB, w1 - jb);  // positions of this batch (uniform)
    float sc[PB][B::QPG], vf[PB][DPL];
    // every slot of the batch is computed (branch-free, so the wave sums interleave);
    // slots past the wave's range are ignored below
    const int pu = p - jb;  // slot of the current position, if it is in this batch
    float kp_[DPL], vp_[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) { kp_[e] = S.kp[lane * DPL + e]; vp_[e] = S.vp[lane * DPL + e]; }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      float kf[DPL];
      widen(kb.k[u], kf);
      widen(kb.v[u], vf[u]);
#pragma unroll
      for (int e = 0; e < DPL; ++e) {  // slots past the range may hold anything, NaN included: zeroed
        kf[e] = u == pu ? kp_[e] : (u < nb ? kf[e] : 0.f);
        vf[u][e] = u == pu ? vp_[e] : (u < nb ? vf[u][e] : 0.f);
      }
#pragma unroll
      for (int h = 0; h < B::QPG; ++h) {
        float d = q[h][0] * kf[0];
#pragma unroll
        for (int e = 1; e < DPL; ++e) d = fmaf(q[h][e], kf[e], d);
        sc[u][h] = d;
      }
    }
    // scores of the batch: lane L holds position u = L / 8 of head h = (L / 4) % 2
    static_assert(PB * B::QPG == 16, "sixteen scores per batch");
    float flat[16];
#pragma unroll
    for (int u = 0; u < PB; ++u)
#pragma unroll
      for (int h = 0; h < B::QPG; ++h) flat[u * B::QPG + h] = sc[u][h];
    const float s_l = transpose_sum<16>(flat, lane);
    const int u_l = lane >> 3, h_l = (lane >> 2) & 1;
    const bool valid = u_l < nb;
    const float sv = valid ? s_l : -INFINITY;
    // batch maximum of the lane's head: over lane bits 3, 4, 5 (the positions)
    float mx = fmaxf(sv, dpp<kRowRor8, 0xf>(sv, sv));
    mx = fmaxf(mx, xor16(mx, lane));
    mx = fmaxf(mx, xor32(mx, lane));
    const float m_l = h_l ? m[1] : m[0];
    const float mn_l = fmaxf(m_l, mx);
    const float w_l = valid ? __expf(sv - mn_l) : 0.f;
    float ws = w_l + dpp<kRowRor8, 0xf>(0.f, w_l);
    ws += xor16(ws, lane);
    ws += xor32(ws, lane);
    if ((lane & 3) == 0) S.attw[wave][lane >> 2] = w_l;
    float aw[16];
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      const f4 t = *reinterpret_cast<const f4*>(&S.attw[wave][i]);
      aw[i] = t.x; aw[i + 1] = t.y; aw[i + 2] = t.z; aw[i + 3] = t.w;
    }
#pragma unroll
    for (int h = 0; h < B::QPG; ++h) {
      const float mn = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mn_l), 4 * h));
      const float wsum = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(ws), 4 * h));
      const float corr = __expf(m[h] - mn);  // 0 while m is still -inf
      ls[h] = fmaf(ls[h], corr, wsum);
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        float a = acc[h][e] * corr;
#pragma unroll
        for (int u = 0; u < PB; ++u) a = fmaf(aw[u * B::QPG + h], vf[u][e], a);
        acc[h][e] = a;
      }
      m[h] = mn;
    }
  };
  // The loads of the next batch, if there is one, are issued before this one is computed;
  // it moves into place after (that copy waits for it, when it is needed anyway), so no
  // load is left in flight past the loop.
  if (w0 < w1) {
    KvBatch<B> cur, nxt;
    if constexpr (PREFETCHED) cur = first;
    else kv_batch_load<B>(R, w0, lane, cur);
    for (int jb = w0;; jb += PB) {
      const bool more = jb + PB < w1;
      if (more) kv_batch_load<B>(R, jb + PB, lane, nxt);
      batch(cur, jb);
      if (!more) break;
      cur = nxt;
    }
  }
  // Nothing of the wave's is in flight now but copies issued an exchange ago.  A wait the
  // compiler sees keeps it from assuming a batch load is still pending further on, where it
  // would wait for it (and for every later copy) before the next GEMV.
  vmem_drain();
#pragma unroll
  for (int h = 0; h < B::QPG; ++h) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) S.wpart[wave][h][2 + lane * DPL + e] = acc[h][e];
    if (lane == 0) {
      S.wpart[wave][h][0] = m[h];
      S.wpart[wave][h][1] = ls[h];
    }
  }
}

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
    auto layer = [&](int l, auto last) -> bool {
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
        if constexpr (decltype(last)::value) {
          if (lm) lm_load<B>(tl, P, lm0, lm1, wave, lane);  // first LM head pass, ahead of the last exchange
        }
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
    for (int l = 0; l + 1 < L; ++l)
      if (!layer(l, std::false_type{})) return;
    if (!layer(L - 1, std::true_type{})) return;

    // LM head: this workgroup's rows, LMR per pass, two passes in flight
    if (lm) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int rb = lm0; rb < lm1; rb += 2 * LMR) {
        TLM t2;
        if (rb + LMR < lm1) lm_load<B>(t2, P, rb + LMR, lm1, wave, lane);
        lm_dot<B>(tl, S.an, rb, lm1, wave, lane, bv, bi);
        if (rb + LMR >= lm1) break;
        if (rb + 2 * LMR < lm1) lm_load<B>(tl, P, rb + 2 * LMR, lm1, wave, lane);
        lm_dot<B>(t2, S.an, rb + LMR, lm1, wave, lane, bv, bi);
      }
      if (lane == 0) { S.wbest_v[wave] = bv; S.wbest_i[wave] = bi; }
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
template <class B>
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
      // this rank's chunk of cache positions: its first batch is loaded now
      const int nc = n_chunks<B>(p);
      const int csz = (p + 1 + nc - 1) / nc;
      const bool attn = grp && r < nc;
      const int c0 = r * csz, c1 = min(p + 1, r * csz + csz);
      KvBatch<B> kb;
      if (attn) attention_prefetch<B>(P, x, l, c0, c1, wave, lane, kb);
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
      dma_part<TGU::TOTAL, 4>(A.gu(l), slotA, 0, wave, lane);  // slot A is free
      if (gather(grp, std::integral_constant<int, B::RQKV>{}, P.xq + (size_t)x * B::RQKV, B::RQKV, tg0 + 0, S.qkv,
                 r * B::T_QKV, (r + 1) * B::T_QKV)) {
        if constexpr (B::BF16) qk_part<B>(S, S.G[gc & 1] + B::H, S.G[gc & 1] + B::H + B::D, P.rms_eps, P.kv_bf16, wave, lane);
      }
      wsync();  // q rotated, k/v of position p in LDS
      if (S.abort_) return;
      if (grp && r == kPerXcd - 1 && wave == kWorkerWaves - 1) write_kv_entry<B>(P, S, x, l, p, lane);
      // attention over the chunk (its cache rows were loaded at the start of the layer; a
      // copy issued before it would be waited for with them)
      if (attn) attention_chunk<B, true>(P, S, x, l, p, c0, c1, wave, lane, kb);
      mark(1);
      wsync();
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
      dma_part<TGU::TOTAL, 4>(A.gu(l), slotA, 3, wave, lane);
      // O partial (slot B)
      if (grp) {
        if constexpr (B::BF16) tile_dot2<B::T_O, B::OC, In::kSplit>(slotB, reinterpret_cast<const float*>(S.ov_hi),
                                                              reinterpret_cast<const float*>(S.ov_lo), 0.f, S.res, wave, lane);
        else tile_dot_lds<B, TO>(slotB, S.ov, S.res, wave, lane);
      }
      mark(1);
      wsync();
      dma_part<TD::TOTAL, 2>(A.down(l), slotB, 0, wave, lane);  // slot B is free
      if (wave < kDmaWaves) wait_vmem_rt(dma_part_count(NI_D, 2, 0, wave));  // gate/up tile landed
      gather(true, std::integral_constant<int, B::H>{}, P.xxa + (size_t)x * B::H, B::H, tg0 + 3, S.xs, r * B::T_O,
             (r + 1) * B::T_O);
      wsync();  // residual after attention, normalised
      if (S.abort_) return;
      dma_part<TD::TOTAL, 2>(A.down(l), slotB, 1, wave, lane);
      // the next layer's gains: their buffer held those of the layer before this one, last
      // read by this layer's q/k/v GEMV
      dma_copy<GCH>(A.gains(ln), S.G[(gc + 1) & 1], wave, lane);
      // gate / up (slot A)
      if constexpr (B::BF16) tile_dot2<B::T_GU, B::H, In::kF32Norm>(slotA, S.xs, S.G[gc & 1], P.rms_eps, S.res, wave, lane);
      else tile_dot_lds<B, TGU>(slotA, S.an, S.res, wave, lane);
      mark(1);
      wsync();
      if (wave < kDmaWaves) wait_vmem_rt(dma_count(NI_GA, wave));  // down tile landed
      gather(true, std::integral_constant<int, B::IX>{}, P.xm + (size_t)x * B::IX, B::IX, tg0 + 4, S.mv,
             r * (B::T_GU / 2), (r + 1) * (B::T_GU / 2));
      wsync();  // SwiGLU slice of the XCD
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
      wsync();  // residual after the MLP, normalised for the next layer or the head
      if (!lm && l + 1 == L) dma_copy<TO::TOTAL>(A.o(0), slotB, wave, lane);  // the next position's layer 0
      ++gc;
      if (S.abort_) return;
    }
    // LM head: this workgroup's rows, LMR per pass, two passes in flight
    if (lm) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int rb = lm0; rb < lm1; rb += 2 * LMR) {
        TLM t2;
        if (rb + LMR < lm1) lm_load<B>(t2, P, rb + LMR, lm1, wave, lane);
        lm_dot<B>(tl, S.an, rb, lm1, wave, lane, bv, bi);
        if (rb + LMR >= lm1) break;
        if (rb + 2 * LMR < lm1) lm_load<B>(tl, P, rb + 2 * LMR, lm1, wave, lane);
        lm_dot<B>(t2, S.an, rb + LMR, lm1, wave, lane, bv, bi);
      }
      if (lane == 0) { S.wbest_v[wave] = bv; S.wbest_i[wave] = bi; }
      wait_vmem<0>();  // next gains and q/k/v tile landed
      dma_copy<TO::TOTAL>(A.o(0), slotB, wave, lane);
      wsync();
    }
  }
}

// ------------------------------------------------------------------ control wave
template <class B>
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
    const uint32_t tag14 = (P.lm_seq0 + (uint32_t)(t - P.logits_from)) & 0x3fffu;
    constexpr int K = kGrid / 64;
    u64 w[K];
    uint32_t pending = (1u << K) - 1;
    uint32_t it = 0;
    const unsigned long long a = wall_clock64();
    while (true) {
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (pending & (1u << k)) w[k] = ld_coh(P.xarg + lane + 64 * k);
#pragma unroll
      for (int k = 0; k < K; ++k)
        if ((pending & (1u << k)) && ((w[k] >> 18) & 0x3fffu) == tag14) pending &= ~(1u << k);
      if (!__any(pending != 0)) break;
      if (++it >= P.spin_limit) {
        if (pending) {
          const int k0 = __builtin_ctz(pending);
          uint32_t seen = 0;
#pragma unroll
          for (int k = 0; k < K; ++k) seen = k == k0 ? (uint32_t)((w[k] >> 18) & 0x3fffu) : seen;
          raise_timeout(P, P.xarg + lane + 64 * k0, tag14, seen);
        }
        fail();
        return false;
      }
      if ((it & 63) == 0 && ld_coh32(P.abort_flag)) { fail(); return false; }
      __builtin_amdgcn_s_sleep(1);
    }
    wait_ticks += wall_clock64() - a;
    u64 best = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) best = w[k] > best ? w[k] : best;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const u64 other = __shfl_xor(best, o);
      best = other > best ? other : best;
    }
    *out_id = 0x3ffff - (int)(best & 0x3ffffu);
    return true;
  };
  // position t's id to the outputs, the pinned id ring and the pinned progress word
  // (workgroup 0 only).  Each ring entry carries its call and lap, so the host tells an
  // entry that is still behind the progress word from a stale one and the two stores need
  // no wait between them.
  auto publish = [&](int t, int id) {
    if (lane == 0) {
      const int slot = t - P.logits_from;
      if (P.out_ids) P.out_ids[slot] = id;
      if (P.pinned_ids)
        __hip_atomic_store(P.pinned_ids + (slot & (kIdRing - 1)), ring_entry(P.call_seq, slot, id), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(P.progress, ((u64)P.call_seq << 32) | (u64)(slot + 1), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
    }
  };
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
        if (id >= P.vocab || (id < 0 && P.rows == nullptr)) {
          if (lane == 0) raise_error(P, DEV_ERR_ID);
          id = 0;
        }
        if (id >= 0) {
          const uint8_t* row = reinterpret_cast<const uint8_t*>(P.embed) + (size_t)id * B::H * B::WB;
          // greedy feedback with rows: the fed-back id's embedding plus row t (the rest of
          // the frame's embeddings, summed by the caller)
          const float* rest = (P.feedback && P.rows) ? P.rows + (size_t)t * B::H : nullptr;
#pragma unroll
          for (int k = 0; k < B::HPL; ++k) {
            const int i = lane + 64 * k;
            const float e = B::BF16 ? bf16_to_f(reinterpret_cast<const uint16_t*>(row)[i])
                                    : reinterpret_cast<const float*>(row)[i];
            S.xs[i] = rest ? e + rest[i] : e;
          }
        } else {
          const float* row = P.rows + (size_t)t * B::H;
#pragma unroll
          for (int k = 0; k < B::HPL; ++k) S.xs[lane + 64 * k] = row[lane + 64 * k];
        }
        if (lane < P.n_sections) {  // a stream outside the rotary table is flagged and read as 0
          const int v = P.pos3 ? P.pos3[t * 3 + lane] : p;
          if (v < 0 || v >= P.rope_positions) raise_error(P, DEV_ERR_POS);
        }
        // cos/sin of every rotary pair at this position (pair i turns with its section's stream)
        for (int i = lane; i < B::D / 2; i += 64) {
          const int sct = i < P.sec_end0 ? 0 : (i < P.sec_end1 ? 1 : 2);
          int ps = P.pos3 ? P.pos3[t * 3 + sct] : p;
          ps = (ps < 0 || ps >= P.rope_positions) ? 0 : ps;
          S.rope_c[i] = P.rope_cos[(size_t)ps * (B::D / 2) + i];
          S.rope_s[i] = P.rope_sin[(size_t)ps * (B::D / 2) + i];
        }
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
      {
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
        if (grp && r < nc) {
          // every wave partial is read first (independent LDS loads), then combined
          float mw[B::QPG][kWorkerWaves], lw[B::QPG][kWorkerWaves], aw[B::QPG][kWorkerWaves][B::DPL];
#pragma unroll
          for (int h = 0; h < B::QPG; ++h)
#pragma unroll
            for (int w = 0; w < kWorkerWaves; ++w) {
              mw[h][w] = S.wpart[w][h][0];
              lw[h][w] = S.wpart[w][h][1];
#pragma unroll
              for (int k = 0; k < B::DPL; ++k) aw[h][w][k] = S.wpart[w][h][2 + lane + 64 * k];
            }
#pragma unroll
          for (int h = 0; h < B::QPG; ++h) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWorkerWaves; ++w) M = fmaxf(M, mw[h][w]);
            float Ls = 0.f;
#pragma unroll
            for (int w = 0; w < kWorkerWaves; ++w) {
              const float f = mw[h][w] == -INFINITY ? 0.f : __expf(mw[h][w] - M);
              Ls = fmaf(lw[h][w], f, Ls);
#pragma unroll
              for (int k = 0; k < B::DPL; ++k) ca[h][k] = fmaf(aw[h][w][k], f, ca[h][k]);
            }
            cM[h] = M;
            cL[h] = Ls;
          }
        }
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
      if (!sync()) return;
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
      if (!sync()) return;
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
      if (!sync()) return;
    }  // layers

    // ---------------------------------------------------------------- argmax key of this workgroup
    if (t >= P.logits_from) {
      sync();  // workers' per-wave best
      float bv = -INFINITY;
      int bi = 0x3ffff;
      for (int w = 0; w < kWorkerWaves; ++w) {
        const float v = S.wbest_v[w];
        const int i = S.wbest_i[w];
        if (i < P.vocab && (v > bv || (v == bv && i < bi))) { bv = v; bi = i; }
      }
      const uint32_t tag14 = (P.lm_seq0 + (uint32_t)(t - P.logits_from)) & 0x3fffu;
      u64 key = ((u64)tag14 << 18) | (u64)(0x3ffff - bi);
      if (bi < P.vocab) key |= (u64)ordered_key(bv) << 32;
      if (lane == 0) __hip_atomic_store(P.xarg + b, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

template <class B>
__device__ __forceinline__ void persistent_body(const Params& P) {
  __shared__ __align__(16) u4 slotA[slot_a_bytes<B>() / 16];
  __shared__ __align__(16) u4 slotB[slot_b_bytes<B>() / 16];
  __shared__ __align__(16) Lds<B> S;
  const int b = blockIdx.x, x = b % kXcds, r = b / kXcds;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (threadIdx.x == 0) S.abort_ = 0;
  if (wave == kWorkerWaves) control_loop<B>(P, S, slotA, slotB, x, r, lane);
  else if constexpr (lds_tiles<B>()) worker_loop_lds<B>(P, S, slotA, slotB, x, r, wave, lane);
  else worker_loop_regs<B>(P, S, x, r, wave, lane);
}

// The same persistent body under two names, so that a profile tells decode launches
// (the LM head at every step) from prompt launches (the LM head at the last position).
template <class B>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(Params P) { persistent_body<B>(P); }
template <class B>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(Params P) { persistent_body<B>(P); }

// Dynamic LDS added to the kernel's static LDS so that a workgroup takes more than half
// of a CU's 160 KB: the grid then places exactly one workgroup on each CU.
template <class B>
static int lds_padding() {
  hipFuncAttributes a;
  if (hipFuncGetAttributes(&a, (const void*)decode_kernel<B>) != hipSuccess) return -1;
  const int need = 80 * 1024 + 1024 - (int)a.sharedSizeBytes;
  return need > 0 ? need : 0;
}

template <class B>
static int launch_t(const Params& p, bool prompt, void* stream) {
  Params pp = p;
  void* args[] = {&pp};
  const int pad = lds_padding<B>();
  if (pad < 0) return -1;
  const void* fn = prompt ? (const void*)prefill_kernel<B> : (const void*)decode_kernel<B>;
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(kGrid), dim3(kThreads), args, (unsigned)pad, (hipStream_t)stream);
  return e == hipSuccess ? 0 : -1;
}

template <class B>
static int coop_t(int* blocks) {
  const int pad = lds_padding<B>();
  if (pad < 0) return -1;
  int nb[2] = {0, 0};
  const void* fns[2] = {(const void*)decode_kernel<B>, (const void*)prefill_kernel<B>};
  for (int k = 0; k < 2; ++k) {
    if (pad > 0 && hipFuncSetAttribute(fns[k], hipFuncAttributeMaxDynamicSharedMemorySize, pad) != hipSuccess) return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb[k], fns[k], kThreads, pad) != hipSuccess) return -1;
  }
  *blocks = nb[0] < nb[1] ? nb[0] : nb[1];
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
