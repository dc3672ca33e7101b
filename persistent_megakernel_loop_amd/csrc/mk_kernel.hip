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
// Workgroup: 8 worker waves hold weight tiles in registers, loaded one layer
// ahead, and do the dot products; one control wave does every exchange.  Worker
// loads never sit in front of a poll in the control wave's in-order load counter.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

namespace mk {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;

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

constexpr int largest_divisor_le8(int r) {
  for (int d = kWorkerWaves; d >= 1; --d)
    if (r % d == 0) return d;
  return 1;
}

// A weight tile: ROWS consecutive rows of COLS columns, contiguous in the arena.
// Wave w < NWA owns rows [w*RPW, (w+1)*RPW); its chunks are read lane-linearly.
template <class B, int ROWS, int COLS>
struct Tile {
  static constexpr int NWA = largest_divisor_le8(ROWS);
  static constexpr int RPW = ROWS / NWA;
  static constexpr int CPR = COLS / B::E;
  static constexpr int CPW = RPW * CPR;
  static constexpr int LPL = (CPW + 63) / 64;
  static constexpr size_t BYTES = (size_t)ROWS * COLS * B::WB;
  static_assert(COLS % B::E == 0, "chunk");
  static_assert(CPR % 64 == 0 || 64 % CPR == 0 || true, "");
  u4 v[LPL];
};

// ------------------------------------------------------------------ small helpers
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// Round to bf16, nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_round(float f) { return bf16_to_f(f_to_bf16(f)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ u64 tagword(float v, uint32_t tag) { return ((u64)tag << 32) | __float_as_uint(v); }
__device__ __forceinline__ void st_tag(u64* p, float v, uint32_t tag) {
  __hip_atomic_store(p, tagword(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_coh(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ void raise_error(const Params& P, uint32_t bits) {
  __hip_atomic_fetch_or(P.err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Control wave: wait until words src[0..n) all carry `tag`, copy their values to dst.
// Returns false if the wait gave up (spin limit or another workgroup's abort).
constexpr int kPollK = 16;  // words in flight per lane per round
__device__ bool poll_words(const u64* src, int n, uint32_t tag, float* dst, int lane, const Params& P) {
  for (int base = 0; base < n; base += 64 * kPollK) {
    const int cnt = min(n - base, 64 * kPollK);
    uint32_t pending = 0;
#pragma unroll
    for (int k = 0; k < kPollK; ++k)
      if (lane + 64 * k < cnt) pending |= 1u << k;
    uint32_t it = 0;
    while (true) {
      u64 w[kPollK];
#pragma unroll
      for (int k = 0; k < kPollK; ++k)
        if (pending & (1u << k)) w[k] = ld_coh(src + base + lane + 64 * k);
#pragma unroll
      for (int k = 0; k < kPollK; ++k)
        if ((pending & (1u << k)) && (uint32_t)(w[k] >> 32) == tag) {
          dst[base + lane + 64 * k] = __uint_as_float((uint32_t)w[k]);
          pending &= ~(1u << k);
        }
      if (!__any(pending != 0)) break;
      if (++it >= P.spin_limit) {
        raise_error(P, DEV_ERR_TIMEOUT);
        __hip_atomic_store(P.abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
      if ((it & 63) == 0 && ld_coh32(P.abort_flag)) return false;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return true;
}

// ------------------------------------------------------------------ GEMV tiles
template <class T>
__device__ __forceinline__ void tile_load(T& t, const uint8_t* base, int wave, int lane) {
  if (wave >= T::NWA) return;
  const u4* p = reinterpret_cast<const u4*>(base) + (size_t)wave * T::CPW;
#pragma unroll
  for (int j = 0; j < T::LPL; ++j) {
    const int k = j * 64 + lane;
    if (T::CPW % 64 == 0 || k < T::CPW) t.v[j] = __builtin_nontemporal_load(p + k);
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
    if (T::CPW % 64 == 0 || k < T::CPW) {
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
    for (int r = 0; r < T::RPW; ++r) res[wave * T::RPW + r] = acc[r];
  }
}

// ------------------------------------------------------------------ the kernel
template <class B>
struct Lds {
  float xs[B::H];            // residual stream (every workgroup holds all of it)
  float an[B::H];            // normalised input of the next GEMV
  float qkv[B::RQKV];        // raw q,k,v of this XCD's group, then q rotated and scaled
  float kp[B::D], vp[B::D];  // K and V of the current position (cache precision)
  float ov[B::OC];           // attention output of the group
  float mv[B::IX];           // SwiGLU output slice
  float res[64];             // row results of the current tile
  float part[kPerXcd][B::QPG][B::D + 2];        // chunk partials read back for the combine
  float wpart[kWorkerWaves][B::QPG][B::D + 2];  // per-wave attention partials
  float wbest_v[kWorkerWaves];
  int wbest_i[kWorkerWaves];
  int streams[3];
  int abort_;
};

__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Attention at position p covers positions 0..p, cut into n_chunks contiguous chunks
// of chunk_len positions; chunk r goes to rank r of the group's XCD.
constexpr int kMinChunk = 32;
__device__ __forceinline__ int n_chunks(int p) { return min(kPerXcd, max(1, (p + 1 + kMinChunk - 1) / kMinChunk)); }

template <class B>
__device__ __forceinline__ void norm_to(const float* x, const float* g, float* out, float eps, int lane) {
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < B::HPL; ++k) { const float v = x[lane + 64 * k]; ss = fmaf(v, v, ss); }
  ss = wave_sum(ss);
  const float rs = rsqrtf(ss / (float)B::H + eps);
#pragma unroll
  for (int k = 0; k < B::HPL; ++k) { const int i = lane + 64 * k; out[i] = g[i] * (x[i] * rs); }
}

// Addresses of this workgroup's tiles in layer l.
template <class B>
struct TileAddr {
  const Params& P;
  int x, r;
  __device__ const uint8_t* layer(int l) const { return P.layers + (size_t)l * P.lay.stride; }
  __device__ const uint8_t* qkv(int l) const {
    return layer(l) + P.lay.qkv + ((size_t)x * B::RQKV + (size_t)r * B::T_QKV) * B::H * B::WB;
  }
  __device__ const uint8_t* o(int l) const {
    return layer(l) + P.lay.o + ((size_t)x * B::H + (size_t)r * B::T_O) * B::OC * B::WB;
  }
  __device__ const uint8_t* gu(int l) const {
    return layer(l) + P.lay.gu + ((size_t)x * kPerXcd + r) * (size_t)B::T_GU * B::H * B::WB;
  }
  __device__ const uint8_t* down(int l) const {
    return layer(l) + P.lay.down + ((size_t)x * B::H + (size_t)r * B::T_D) * B::IX * B::WB;
  }
  __device__ const float* gain(int l, size_t off) const { return reinterpret_cast<const float*>(layer(l) + off); }
};

// Bodies whose four tiles fit in registers together are loaded a whole layer ahead;
// the larger body loads each tile one phase ahead.
template <class B>
constexpr bool layer_ahead() { return B::H <= 1024; }

// ------------------------------------------------------------------ worker waves
template <class B>
__device__ void worker_loop(const Params& P, Lds<B>& S, int x, int r, int wave, int lane) {
  using TQKV = Tile<B, B::T_QKV, B::H>;
  using TO = Tile<B, B::T_O, B::OC>;
  using TGU = Tile<B, B::T_GU, B::H>;
  using TD = Tile<B, B::T_D, B::IX>;
  using TLM = Tile<B, 16, B::H>;
  const TileAddr<B> A{P, x, r};
  const bool grp = x < B::NG;
  const int L = P.n_layers;
  const int b = blockIdx.x;
  constexpr bool LA = layer_ahead<B>();

  TQKV tq;
  TO to;
  TGU tg;
  TD td;
  if (grp) tile_load(tq, A.qkv(0), wave, lane);
  if constexpr (LA) {
    if (grp) tile_load(to, A.o(0), wave, lane);
    tile_load(tg, A.gu(0), wave, lane);
    tile_load(td, A.down(0), wave, lane);
  }

  for (int t = 0; t < P.n_pos; ++t) {
    const int p = P.pos0 + t;
    const bool last_t = t + 1 == P.n_pos;
    __syncthreads();  // input fetched
    if (S.abort_) return;
    for (int l = 0; l < L; ++l) {
      const bool more = (l + 1 < L) || !last_t;
      const int ln = (l + 1 < L) ? l + 1 : 0;
      // q, k, v rows
      if (grp) {
        tile_dot<B>(tq, S.an, S.res, wave, lane);
        if constexpr (LA) { if (more) tile_load(tq, A.qkv(ln), wave, lane); }
        else tile_load(to, A.o(l), wave, lane);
      }
      __syncthreads();
      __syncthreads();  // q rotated, k/v of position p in LDS
      if (S.abort_) return;
      // attention over this rank's chunk of positions
      const int nc = n_chunks(p);
      const int csz = (p + 1 + nc - 1) / nc;
      if (grp && r < nc) {
        const int c0 = r * csz, c1 = min(p + 1, c0 + csz);
        float m[B::QPG], ls[B::QPG], acc[B::QPG][B::DPL];
#pragma unroll
        for (int h = 0; h < B::QPG; ++h) {
          m[h] = -INFINITY;
          ls[h] = 0.f;
#pragma unroll
          for (int k = 0; k < B::DPL; ++k) acc[h][k] = 0.f;
        }
        const size_t cbase = (((size_t)l * B::NKV + x) * P.max_seq) * B::D;
        for (int j = c0 + wave; j < c1; j += kWorkerWaves) {
          float kk[B::DPL], vv[B::DPL];
          if (j == p) {
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) { kk[k] = S.kp[lane + 64 * k]; vv[k] = S.vp[lane + 64 * k]; }
          } else {
            const size_t off = cbase + (size_t)j * B::D;
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) {
              const int i = lane + 64 * k;
              if (P.kv_bf16) {
                kk[k] = bf16_to_f(__hip_atomic_load(reinterpret_cast<const uint16_t*>(P.kcache) + off + i,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                vv[k] = bf16_to_f(__hip_atomic_load(reinterpret_cast<const uint16_t*>(P.vcache) + off + i,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
              } else {
                kk[k] = __hip_atomic_load(reinterpret_cast<const float*>(P.kcache) + off + i, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                vv[k] = __hip_atomic_load(reinterpret_cast<const float*>(P.vcache) + off + i, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
              }
            }
          }
#pragma unroll
          for (int h = 0; h < B::QPG; ++h) {
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) s = fmaf(S.qkv[h * B::D + lane + 64 * k], kk[k], s);
            s = wave_sum(s);
            const float mn = fmaxf(m[h], s);
            const float corr = __expf(m[h] - mn);
            const float e = __expf(s - mn);
            ls[h] = ls[h] * corr + e;
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) acc[h][k] = fmaf(acc[h][k], corr, e * vv[k]);
            m[h] = mn;
          }
        }
#pragma unroll
        for (int h = 0; h < B::QPG; ++h) {
#pragma unroll
          for (int k = 0; k < B::DPL; ++k) S.wpart[wave][h][2 + lane + 64 * k] = acc[h][k];
          if (lane == 0) {
            S.wpart[wave][h][0] = m[h];
            S.wpart[wave][h][1] = ls[h];
          }
        }
      }
      __syncthreads();
      __syncthreads();  // attention output of the group in LDS
      if (S.abort_) return;
      // O partial
      if (grp) {
        tile_dot<B>(to, S.ov, S.res, wave, lane);
        if constexpr (LA) { if (more) tile_load(to, A.o(ln), wave, lane); }
      }
      if constexpr (!LA) tile_load(tg, A.gu(l), wave, lane);
      __syncthreads();
      __syncthreads();  // residual after attention, normalised
      if (S.abort_) return;
      // gate / up
      tile_dot<B>(tg, S.an, S.res, wave, lane);
      if constexpr (LA) { if (more) tile_load(tg, A.gu(ln), wave, lane); }
      else tile_load(td, A.down(l), wave, lane);
      __syncthreads();
      __syncthreads();  // SwiGLU slice of the XCD
      if (S.abort_) return;
      // down partial
      tile_dot<B>(td, S.mv, S.res, wave, lane);
      if constexpr (LA) { if (more) tile_load(td, A.down(ln), wave, lane); }
      else if (grp && more) tile_load(tq, A.qkv(ln), wave, lane);
      __syncthreads();
      __syncthreads();  // residual after the MLP, normalised for the next layer or the head
      if (S.abort_) return;
    }
    // LM head rows of this workgroup, 16 rows per pass, best (value, lowest row) per wave
    if (t >= P.logits_from) {
      const int rpb = (P.vocab + kGrid - 1) / kGrid;
      const int row0 = b * rpb, row1 = min(P.vocab, row0 + rpb);
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      TLM tl;
      for (int rb = row0; rb < row1; rb += 16) {
        const int myrow0 = rb + wave * TLM::RPW;
        const u4* pp = reinterpret_cast<const u4*>(reinterpret_cast<const uint8_t*>(P.lm_head) +
                                                    (size_t)rb * B::H * B::WB) + (size_t)wave * TLM::CPW;
#pragma unroll
        for (int j = 0; j < TLM::LPL; ++j) {
          const int k = j * 64 + lane;
          const int row = myrow0 + k / TLM::CPR;
          if (k < TLM::CPW && row < row1) tl.v[j] = __builtin_nontemporal_load(pp + k);
          else tl.v[j] = u4{0, 0, 0, 0};
        }
        float acc[TLM::RPW];
#pragma unroll
        for (int q = 0; q < TLM::RPW; ++q) acc[q] = 0.f;
#pragma unroll
        for (int j = 0; j < TLM::LPL; ++j) {
          const int k = j * 64 + lane;
          if (k < TLM::CPW) {
            const int row = k / TLM::CPR;
            const float d = dot_chunk<B>(tl.v[j], S.an + (k - row * TLM::CPR) * B::E);
#pragma unroll
            for (int q = 0; q < TLM::RPW; ++q) acc[q] += (row == q) ? d : 0.f;
          }
        }
#pragma unroll
        for (int q = 0; q < TLM::RPW; ++q) {
          const float v = wave_sum(acc[q]);
          const int row = myrow0 + q;
          if (row < row1 && (v > bv || (v == bv && row < bi))) { bv = v; bi = row; }
        }
      }
      if (lane == 0) { S.wbest_v[wave] = bv; S.wbest_i[wave] = bi; }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ control wave
template <class B>
__device__ void control_loop(const Params& P, Lds<B>& S, int x, int r, int lane) {
  const TileAddr<B> A{P, x, r};
  const bool grp = x < B::NG;
  const int L = P.n_layers;
  const int b = blockIdx.x;
  const uint32_t tpp = tags_per_position(L);
  const float eps = P.rms_eps;
  const float qscale = rsqrtf((float)B::D);
  unsigned long long wait_ticks = 0, t_start = 0;

  auto fail = [&]() { if (lane == 0) S.abort_ = 1; };
  auto abort_all = [&]() {
    raise_error(P, DEV_ERR_TIMEOUT);
    __hip_atomic_store(P.abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto timed_poll = [&](const u64* src, int n, uint32_t tag, float* dst) {
    const unsigned long long a = wall_clock64();
    const bool ok = poll_words(src, n, tag, dst, lane, P);
    wait_ticks += wall_clock64() - a;
    if (!ok) fail();
    return ok;
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
      if (++it >= P.spin_limit) { abort_all(); fail(); return false; }
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
  // position t's id to the outputs and the pinned progress word (workgroup 0 only)
  auto publish = [&](int t, int id) {
    if (lane == 0) {
      const int slot = t - P.logits_from;
      if (P.out_ids) P.out_ids[slot] = id;
      if (P.pinned_ids) __hip_atomic_store(P.pinned_ids + slot, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __builtin_amdgcn_s_waitcnt(0);
      __hip_atomic_store(P.progress, ((u64)P.call_seq << 32) | (u64)(slot + 1), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
    }
  };
  auto sync = [&]() { __syncthreads(); return S.abort_ == 0; };

  int pending_lm = -1;  // position whose LM head ran and whose id is not published yet
  for (int t = 0; t < P.n_pos; ++t) {
    const int p = P.pos0 + t;
    const uint32_t tbase = P.tag0 + (uint32_t)t * tpp;
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
#pragma unroll
          for (int k = 0; k < B::HPL; ++k) {
            const int i = lane + 64 * k;
            S.xs[i] = B::BF16 ? bf16_to_f(reinterpret_cast<const uint16_t*>(row)[i])
                              : reinterpret_cast<const float*>(row)[i];
          }
        } else {
          const float* row = P.rows + (size_t)t * B::H;
#pragma unroll
          for (int k = 0; k < B::HPL; ++k) S.xs[lane + 64 * k] = row[lane + 64 * k];
        }
        if (lane < 3) {
          int v = P.pos3 ? P.pos3[t * 3 + lane] : p;
          if (v < 0 || v >= P.rope_positions) {
            if (lane < P.n_sections) raise_error(P, DEV_ERR_POS);
            v = 0;
          }
          S.streams[lane] = v;
        }
        norm_to<B>(S.xs, A.gain(0, P.lay.in_norm), S.an, eps, lane);
        if (P.dbg_hidden && b == 0)
          for (int k = 0; k < B::HPL; ++k)
            P.dbg_hidden[((size_t)t * (L + 1)) * B::H + lane + 64 * k] = S.xs[lane + 64 * k];
      }
    }
    if (!sync()) return;

    for (int l = 0; l < L; ++l) {
      const uint32_t tg0 = tbase + (uint32_t)l * kPhasesPerLayer;
      // ------------------------------------------------------------ q,k,v of the group
      if (!sync()) return;
      if (grp) {
        u64* xq = P.xq + (size_t)x * B::RQKV;
        if (lane < B::T_QKV) st_tag(xq + r * B::T_QKV + lane, S.res[lane], tg0 + 0);
        if (timed_poll(xq, B::RQKV, tg0 + 0, S.qkv)) {
          // per-head RMSNorm of q and k, rotation, rounding of the cache entry
          const float* qn = A.gain(l, P.lay.q_norm);
          const float* kn = A.gain(l, P.lay.k_norm);
          for (int h = 0; h <= B::QPG; ++h) {  // h == QPG is k
            float* v = S.qkv + h * B::D;
            const float* g = h < B::QPG ? qn : kn;
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) { const float a = v[lane + 64 * k]; ss = fmaf(a, a, ss); }
            ss = wave_sum(ss);
            const float rs = rsqrtf(ss / (float)B::D + eps);
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) { const int i = lane + 64 * k; v[i] = g[i] * (v[i] * rs); }
            // LDS accesses of one wave are performed in order: the lane owning pair i
            // sees every lane's normalised value
            for (int i = lane; i < B::D / 2; i += 64) {
              const int s = i < P.sec_end0 ? 0 : (i < P.sec_end1 ? 1 : 2);
              const int ps = S.streams[s];
              const float c = P.rope_cos[(size_t)ps * (B::D / 2) + i];
              const float sn = P.rope_sin[(size_t)ps * (B::D / 2) + i];
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
#pragma unroll
          for (int k = 0; k < B::DPL; ++k) {
            const int i = lane + 64 * k;
            const float v = S.qkv[(B::QPG + 1) * B::D + i];
            S.vp[i] = P.kv_bf16 ? bf16_round(v) : v;
          }
          if (r == 0) {  // the group's cache entry at position p
            const size_t off = (((size_t)l * B::NKV + x) * P.max_seq + p) * B::D;
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) {
              const int i = lane + 64 * k;
              if (P.kv_bf16) {
                __hip_atomic_store(reinterpret_cast<uint16_t*>(P.kcache) + off + i, f_to_bf16(S.kp[i]),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(reinterpret_cast<uint16_t*>(P.vcache) + off + i, f_to_bf16(S.vp[i]),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              } else {
                __hip_atomic_store(reinterpret_cast<float*>(P.kcache) + off + i, S.kp[i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(reinterpret_cast<float*>(P.vcache) + off + i, S.vp[i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
              }
            }
          }
        }
      }
      if (!sync()) return;
      // ------------------------------------------------------------ attention combine
      if (!sync()) return;
      if (grp) {
        const int nc = n_chunks(p);
        u64* xa = P.xatt + (size_t)x * kPerXcd * B::QPG * (B::D + 2);
        if (r < nc) {
          // merge the 8 waves' partials, fixed order, into this chunk's partial
          for (int h = 0; h < B::QPG; ++h) {
            float M = -INFINITY;
            for (int w = 0; w < kWorkerWaves; ++w) M = fmaxf(M, S.wpart[w][h][0]);
            float Ls = 0.f, a[B::DPL];
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) a[k] = 0.f;
            for (int w = 0; w < kWorkerWaves; ++w) {
              const float mw = S.wpart[w][h][0];
              const float f = mw == -INFINITY ? 0.f : __expf(mw - M);
              Ls = fmaf(S.wpart[w][h][1], f, Ls);
#pragma unroll
              for (int k = 0; k < B::DPL; ++k) a[k] = fmaf(S.wpart[w][h][2 + lane + 64 * k], f, a[k]);
            }
            u64* dst = xa + ((size_t)r * B::QPG + h) * (B::D + 2);
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) st_tag(dst + 2 + lane + 64 * k, a[k], tg0 + 1);
            if (lane == 0) {
              st_tag(dst, M, tg0 + 1);
              st_tag(dst + 1, Ls, tg0 + 1);
            }
          }
        }
        if (timed_poll(xa, nc * B::QPG * (B::D + 2), tg0 + 1, &S.part[0][0][0])) {
          for (int h = 0; h < B::QPG; ++h) {
            float M = -INFINITY;
            for (int c = 0; c < nc; ++c) M = fmaxf(M, S.part[c][h][0]);
            float Ls = 0.f, a[B::DPL];
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) a[k] = 0.f;
            for (int c = 0; c < nc; ++c) {
              const float mc = S.part[c][h][0];
              const float f = mc == -INFINITY ? 0.f : __expf(mc - M);
              Ls = fmaf(S.part[c][h][1], f, Ls);
#pragma unroll
              for (int k = 0; k < B::DPL; ++k) a[k] = fmaf(S.part[c][h][2 + lane + 64 * k], f, a[k]);
            }
            const float inv = 1.f / Ls;
#pragma unroll
            for (int k = 0; k < B::DPL; ++k) S.ov[h * B::D + lane + 64 * k] = a[k] * inv;
          }
        }
      }
      if (!sync()) return;
      // ------------------------------------------------------------ O partials -> residual
      if (!sync()) return;
      {
        // group x's partial of rows [r*T_O, (r+1)*T_O) goes to slot [r][x]: the reader of
        // those rows finds every group's partial in one contiguous run
        if (grp && lane < B::T_O) st_tag(P.xop + ((size_t)r * B::NG + x) * B::T_O + lane, S.res[lane], tg0 + 2);
        if (timed_poll(P.xop + (size_t)r * B::NG * B::T_O, B::NG * B::T_O, tg0 + 2, &S.part[0][0][0])) {
          if (lane < B::T_O) {
            float d = 0.f;
            for (int g = 0; g < B::NG; ++g) d += (&S.part[0][0][0])[g * B::T_O + lane];
            st_tag(P.xxa + (size_t)x * B::H + r * B::T_O + lane, S.xs[r * B::T_O + lane] + d, tg0 + 3);
          }
          if (timed_poll(P.xxa + (size_t)x * B::H, B::H, tg0 + 3, S.xs))
            norm_to<B>(S.xs, A.gain(l, P.lay.post_norm), S.an, eps, lane);
        }
      }
      if (!sync()) return;
      // ------------------------------------------------------------ SwiGLU slice
      if (!sync()) return;
      {
        constexpr int HALF = B::T_GU / 2;
        if (lane < HALF) {
          const float gt = S.res[lane], up = S.res[HALF + lane];
          st_tag(P.xm + (size_t)x * B::IX + r * HALF + lane, gt / (1.f + __expf(-gt)) * up, tg0 + 4);
        }
        timed_poll(P.xm + (size_t)x * B::IX, B::IX, tg0 + 4, S.mv);
      }
      if (!sync()) return;
      // ------------------------------------------------------------ down partials -> residual
      if (!sync()) return;
      {
        if (lane < B::T_D) st_tag(P.xdp + ((size_t)r * kXcds + x) * B::T_D + lane, S.res[lane], tg0 + 5);
        if (timed_poll(P.xdp + (size_t)r * kXcds * B::T_D, kXcds * B::T_D, tg0 + 5, &S.part[0][0][0])) {
          if (lane < B::T_D) {
            float d = 0.f;
            for (int g = 0; g < kXcds; ++g) d += (&S.part[0][0][0])[g * B::T_D + lane];
            st_tag(P.xxb + (size_t)x * B::H + r * B::T_D + lane, S.xs[r * B::T_D + lane] + d, tg0 + 6);
          }
          if (timed_poll(P.xxb + (size_t)x * B::H, B::H, tg0 + 6, S.xs)) {
            const float* g = (l + 1 < L) ? A.gain(l + 1, P.lay.in_norm) : P.final_norm;
            norm_to<B>(S.xs, g, S.an, eps, lane);
            if (P.dbg_hidden && b == 0)
              for (int k = 0; k < B::HPL; ++k)
                P.dbg_hidden[((size_t)t * (L + 1) + l + 1) * B::H + lane + 64 * k] = S.xs[lane + 64 * k];
          }
        }
      }
      if (!sync()) return;
    }  // layers

    // ---------------------------------------------------------------- argmax key of this workgroup
    if (t >= P.logits_from) {
      __syncthreads();  // workers' per-wave best
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
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(Params P) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  Lds<B>& S = *reinterpret_cast<Lds<B>*>(lds_raw);
  const int b = blockIdx.x, x = b % kXcds, r = b / kXcds;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x == 0) S.abort_ = 0;
  if (wave == kWorkerWaves) control_loop<B>(P, S, x, r, lane);
  else worker_loop<B>(P, S, x, r, wave, lane);
}

// ------------------------------------------------------------------ small kernels
__global__ void widen_kernel(const void* src, float* dst, int n, int bf16) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = bf16 ? bf16_to_f(reinterpret_cast<const uint16_t*>(src)[i]) : reinterpret_cast<const float*>(src)[i];
}

// Row t: sum of n_cb codebook rows and one text row, float32, one add per row in order.
__global__ void embed_sum_kernel(const void* cb, int n_cb, int cb_size, const void* text, int text_vocab,
                                 int hidden, int bf16, const int32_t* ids, float* rows, int32_t* bad) {
  const int t = blockIdx.x;
  const int32_t* id = ids + (size_t)t * (n_cb + 1);
  for (int i = threadIdx.x; i < hidden; i += blockDim.x) {
    float acc = 0.f;
    for (int c = 0; c <= n_cb; ++c) {
      int v = id[c];
      const int lim = c < n_cb ? cb_size : text_vocab;
      if (v < 0 || v >= lim) { if (i == 0 && bad) atomicAdd(bad, 1); v = 0; }
      const size_t off = c < n_cb ? (((size_t)c * cb_size + v) * hidden + i) : ((size_t)v * hidden + i);
      const void* base = c < n_cb ? cb : text;
      const float w = bf16 ? bf16_to_f(reinterpret_cast<const uint16_t*>(base)[off]) : reinterpret_cast<const float*>(base)[off];
      acc = (c == 0) ? w : acc + w;
    }
    rows[(size_t)t * hidden + i] = acc;
  }
}

template <class B>
static int launch_t(const Params& p, void* stream) {
  Params pp = p;
  void* args[] = {&pp};
  hipError_t e = hipLaunchCooperativeKernel((const void*)decode_kernel<B>, dim3(kGrid), dim3(kThreads), args,
                                            kLdsBytes, (hipStream_t)stream);
  return e == hipSuccess ? 0 : -1;
}

template <class B>
static int coop_t(int* blocks) {
  static_assert(sizeof(Lds<B>) <= (size_t)kLdsBytes, "LDS plan");
  if (hipFuncSetAttribute((const void*)decode_kernel<B>, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) != hipSuccess)
    return -1;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, decode_kernel<B>, kThreads, kLdsBytes) == hipSuccess ? 0 : -1;
}

int launch_decode(int body, const Params& p, void* stream) {
  switch (body) {
    case BODY_TINY: return launch_t<BodyTiny>(p, stream);
    case BODY_Q06: return launch_t<BodyQ06>(p, stream);
    case BODY_Q17: return launch_t<BodyQ17>(p, stream);
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

int launch_embed_sum(const void* codebooks, int n_cb, int cb_size, const void* text, int text_vocab, int hidden,
                     int bf16, const int32_t* ids, int n, float* rows, int32_t* bad, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(embed_sum_kernel, dim3(n), dim3(256), 0, (hipStream_t)stream, codebooks, n_cb, cb_size, text,
                     text_vocab, hidden, bf16, ids, rows, bad);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_widen(const void* src, float* dst, int n, int bf16, void* stream) {
  hipLaunchKernelGGL(widen_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, src, dst, n, bf16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mk
