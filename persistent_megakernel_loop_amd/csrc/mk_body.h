// Device code shared by the persistent kernel and the launch-per-phase kernels: body
// shapes, weight tiles, the LDS layout of a workgroup, the GEMV, norm, rotation,
// attention and LM-head steps of a decode position.  Included by one translation unit
// each; everything here is inline or a template.
#pragma once
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
    // bf16 bodies: the current position's k and v as the cache word they will be (the
    // values are bf16 already, so packing is exact), chosen before widening: one select
    // per word instead of one per element
    uint32_t kpw = 0, vpw = 0;
    if constexpr (B::BF16) {
      kpw = pack_bf16(kp_[0], kp_[1]);
      vpw = pack_bf16(vp_[0], vp_[1]);
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      float kf[DPL];
      if constexpr (B::BF16) {
        // slots past the range may hold anything, NaN included: their values are zeroed;
        // their keys need not be, as their scores are replaced by -inf below
        widen(u == pu ? kpw : kb.k[u], kf);
        widen(u == pu ? vpw : (u < nb ? kb.v[u] : 0u), vf[u]);
      } else {
        widen(kb.k[u], kf);
        widen(kb.v[u], vf[u]);
#pragma unroll
        for (int e = 0; e < DPL; ++e) {  // slots past the range may hold anything, NaN included: zeroed
          kf[e] = u == pu ? kp_[e] : (u < nb ? kf[e] : 0.f);
          vf[u][e] = u == pu ? vp_[e] : (u < nb ? vf[u][e] : 0.f);
        }
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

// ------------------------------------------------------------------ steps of a position
// Row x of the decoder's input at position t (xs, all H; lane takes elements lane + 64k):
// the embedding of `id`, plus row t of P.rows when greedy feedback comes with rows (the
// rest of the frame's embeddings, summed by the caller); a negative id reads row t of
// P.rows.  An id past the vocabulary, or a negative one with no rows, is flagged and read
// as 0.
template <class B>
__device__ __forceinline__ void input_row(const Params& P, float* xs, int t, int id, int lane) {
  if (id >= P.vocab || (id < 0 && P.rows == nullptr)) {
    if (lane == 0) raise_error(P, DEV_ERR_ID);
    id = 0;
  }
  if (id >= 0) {
    const uint8_t* row = reinterpret_cast<const uint8_t*>(P.embed) + (size_t)id * B::H * B::WB;
    const float* rest = (P.feedback && P.rows) ? P.rows + (size_t)t * B::H : nullptr;
#pragma unroll
    for (int k = 0; k < B::HPL; ++k) {
      const int i = lane + 64 * k;
      const float e = B::BF16 ? bf16_to_f(reinterpret_cast<const uint16_t*>(row)[i])
                              : reinterpret_cast<const float*>(row)[i];
      xs[i] = rest ? e + rest[i] : e;
    }
  } else {
    const float* row = P.rows + (size_t)t * B::H;
#pragma unroll
    for (int k = 0; k < B::HPL; ++k) xs[lane + 64 * k] = row[lane + 64 * k];
  }
}

// cos/sin of every rotary pair at position t (pair i turns with its section's stream, the
// position itself without streams); a stream outside the rotary table is flagged and
// read as 0.
template <class B>
__device__ __forceinline__ void rope_row(const Params& P, Lds<B>& S, int t, int p, int lane) {
  if (lane < P.n_sections) {
    const int v = P.pos3 ? P.pos3[t * 3 + lane] : p;
    if (v < 0 || v >= P.rope_positions) raise_error(P, DEV_ERR_POS);
  }
  for (int i = lane; i < B::D / 2; i += 64) {
    const int sct = i < P.sec_end0 ? 0 : (i < P.sec_end1 ? 1 : 2);
    int ps = P.pos3 ? P.pos3[t * 3 + sct] : p;
    ps = (ps < 0 || ps >= P.rope_positions) ? 0 : ps;
    S.rope_c[i] = P.rope_cos[(size_t)ps * (B::D / 2) + i];
    S.rope_s[i] = P.rope_sin[(size_t)ps * (B::D / 2) + i];
  }
}

// The greedy id of position t from every workgroup's LM-head key (float bits, a 14-bit
// sequence number of the LM head, the inverted row index): waits until all carry this
// position's sequence number, then takes the largest.  False if the wait gave up (the
// timeout is recorded) or another workgroup aborted.  Adds the wait to wait_ticks.
__device__ __forceinline__ bool argmax_keys(const Params& P, int t, int lane, int* out_id,
                                            unsigned long long& wait_ticks) {
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
      return false;
    }
    if ((it & 63) == 0 && ld_coh32(P.abort_flag)) return false;
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
}

// This rank's chunk partial of the attention: the worker waves' partials (S.wpart) merged
// in wave order, per query head the running maximum cM, the weight sum cL and the
// weighted value sum ca (lane holds head dims lane + 64k).
template <class B>
__device__ __forceinline__ void merge_wave_partials(const Lds<B>& S, int lane, float (&cM)[B::QPG], float (&cL)[B::QPG],
                                                    float (&ca)[B::QPG][B::DPL]) {
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

// Position t's id to the outputs, the pinned id ring and the pinned progress word (lane 0
// of the caller).  Each ring entry carries its call and lap, so the host tells an entry
// that is still behind the progress word from a stale one and the two stores need no
// wait between them.
__device__ __forceinline__ void publish_id(const Params& P, int t, int id, int lane) {
  if (lane == 0) {
    const int slot = t - P.logits_from;
    if (P.out_ids) P.out_ids[slot] = id;
    if (P.pinned_ids)
      __hip_atomic_store(P.pinned_ids + (slot & (kIdRing - 1)), ring_entry(P.call_seq, slot, id), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(P.progress, ((u64)P.call_seq << 32) | (u64)(slot + 1), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// LM head rows [lm0, lm1) of this workgroup on the final-normalised input S.an: worker
// wave `wave` takes two rows of every pass of 2 x 7 rows, two passes in flight (the
// first one's loads in tl, issued by the caller); its best (value, lowest row) goes to
// S.wbest_v/i[wave].
template <class B, class T>
__device__ __forceinline__ void lm_rows(const Params& P, Lds<B>& S, T& tl, int lm0, int lm1, int wave, int lane) {
  constexpr int LMR = 2 * kWorkerWaves;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int rb = lm0; rb < lm1; rb += 2 * LMR) {
    T t2;
    if (rb + LMR < lm1) lm_load<B>(t2, P, rb + LMR, lm1, wave, lane);
    lm_dot<B>(tl, S.an, rb, lm1, wave, lane, bv, bi);
    if (rb + LMR >= lm1) break;
    if (rb + 2 * LMR < lm1) lm_load<B>(tl, P, rb + 2 * LMR, lm1, wave, lane);
    lm_dot<B>(t2, S.an, rb + LMR, lm1, wave, lane, bv, bi);
  }
  if (lane == 0) { S.wbest_v[wave] = bv; S.wbest_i[wave] = bi; }
}

// The workgroup's LM-head key of position t from the waves' bests: float bits (ordered),
// the LM head's 14-bit sequence number, the inverted row (ties: lowest row), stored to
// xarg[b] for every workgroup's argmax_keys.
template <class B>
__device__ __forceinline__ void publish_lm_key(const Params& P, const Lds<B>& S, int t, int b, int lane) {
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
}

}  // namespace mk
