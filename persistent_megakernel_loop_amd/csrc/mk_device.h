// Device-side helpers shared by the persistent decode bodies: wave reductions (DPP and
// lane-half swaps), bf16 conversions and the split-input dot products, the tagged-word
// exchange every cross-workgroup hop uses, and the LDS DMA copy with its explicit waits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "mk_internal.h"

namespace mk {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;

// ------------------------------------------------------------------ small helpers
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// Round to bf16, nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f_to_bf16(float f) {
  const __bf16 b = (__bf16)f;  // the conversion instruction: round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float bf16_round(float f) { return bf16_to_f(f_to_bf16(f)); }

// Cross-lane reductions with DPP (data-parallel primitives of the vector ALU) instead of
// LDS permutes: xor-1 and xor-2 quad permutes, half-row and row mirrors (16-lane sums),
// then row broadcasts that fold rows 0..3 into lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
constexpr int kQuadXor1 = 0xb1, kQuadXor2 = 0x4e, kRowHalfMirror = 0x141, kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143, kRowRor8 = 0x128;

// Sum over each group of 16 lanes, in every lane of the group.
__device__ __forceinline__ float sum16(float v) {
  v += dpp<kQuadXor1, 0xf>(0.f, v);
  v += dpp<kQuadXor2, 0xf>(0.f, v);
  v += dpp<kRowHalfMirror, 0xf>(0.f, v);
  v += dpp<kRowMirror, 0xf>(0.f, v);
  return v;
}
// Sum over groups of G consecutive lanes (G a power of two up to 32); the total sits in
// the group's last lane.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp<kQuadXor1, 0xf>(0.f, v);
  if constexpr (G >= 4) v += dpp<kQuadXor2, 0xf>(0.f, v);
  if constexpr (G >= 8) v += dpp<kRowHalfMirror, 0xf>(0.f, v);
  if constexpr (G >= 16) v += dpp<kRowMirror, 0xf>(0.f, v);
  if constexpr (G >= 32) v += dpp<kRowBcast15, 0xa>(0.f, v);
  return v;
}

// Sum over the wave, returned to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  v += dpp<kRowBcast15, 0xa>(0.f, v);  // rows 1, 3 += last lane of rows 0, 2
  v += dpp<kRowBcast31, 0xc>(0.f, v);  // rows 2, 3 += last lane of row 1
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kQuadXor1, 0xf>(v, v));
  v = fmaxf(v, dpp<kQuadXor2, 0xf>(v, v));
  v = fmaxf(v, dpp<kRowHalfMirror, 0xf>(v, v));
  v = fmaxf(v, dpp<kRowMirror, 0xf>(v, v));
  v = fmaxf(v, dpp<kRowBcast15, 0xa>(v, v));
  v = fmaxf(v, dpp<kRowBcast31, 0xc>(v, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Value of lane ^ 16 and of lane ^ 32, through the row-swap instructions (no LDS).
__device__ __forceinline__ float xor16(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(((lane >> 4) & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(lane >= 32 ? r[0] : r[1]);
}

// N wave sums at once (N = 2, 4, 8 or 16): lane L returns the sum over the wave of
// v[L / (64 / N)] (for N = 2 only in the last lane of each half).  Each butterfly stage
// pairs two values and keeps, in each half of the lanes, the partial sum of one of them:
// lane-half swaps for the 32- and 16-lane steps, DPP for 8 and 4, then the sum within
// the remaining 64 / N lanes.  Sixteen sums cost about as much as two single ones.
template <int N>
__device__ __forceinline__ float transpose_sum(const float (&v)[N], int lane) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "lane groups");
  float a[N];
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] = v[i];
  int n = N;
  // lane bit 5: lanes < 32 keep a[i], the others a[i + n/2]
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[i]), __float_as_uint(a[i + N / 2]), false, false);
    a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  n = N / 2;
  if constexpr (N >= 4) {  // lane bit 4: even rows keep a[i], odd rows a[i + n/2]
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]), __float_as_uint(a[i + N / 4]), false, false);
      a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }
  if constexpr (N >= 8) {  // lane bit 3
    const bool b3 = (lane & 8) != 0;
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const float send = b3 ? a[i] : a[i + N / 8];
      a[i] = (b3 ? a[i + N / 8] : a[i]) + dpp<kRowRor8, 0xf>(0.f, send);  // lane ^ 8 within the row
    }
  }
  if constexpr (N >= 16) {  // lane bit 2: lanes 0-3 <-> 7-4 of each eight
    const bool b2 = (lane & 4) != 0;
    const float send = b2 ? a[0] : a[1];
    a[0] = (b2 ? a[1] : a[0]) + dpp<kRowHalfMirror, 0xf>(0.f, send);
  }
  float z = a[0];
  if constexpr (N == 16) {
    z += dpp<kQuadXor1, 0xf>(0.f, z);
    z += dpp<kQuadXor2, 0xf>(0.f, z);
  } else if constexpr (N == 8) {
    z += dpp<kRowHalfMirror, 0xf>(0.f, z);
    z += dpp<kQuadXor1, 0xf>(0.f, z);
    z += dpp<kQuadXor2, 0xf>(0.f, z);
  } else if constexpr (N == 4) {
    z = sum16(z);
  } else {
    z = group_sum<32>(z);
  }
  (void)n;
  return z;
}

__device__ __forceinline__ u64 tagword(float v, uint32_t tag) { return ((u64)tag << 32) | __float_as_uint(v); }
// Cross-XCD words are written through to the device coherence point.
__device__ __forceinline__ void st_tag(u64* p, float v, uint32_t tag) {
  __hip_atomic_store(p, tagword(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Words read only inside the writer's XCD: a plain store that stays in the XCD's L2,
// where the readers' device-coherent loads find it.  Only used once the launch has
// checked that every workgroup runs on XCD b % 8; otherwise written through too.
__device__ __forceinline__ void st_local(u64* p, float v, uint32_t tag, bool plain) {
  if (plain) __hip_atomic_store(p, tagword(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
  else __hip_atomic_store(p, tagword(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_coh(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void raise_error(const Params& P, uint32_t bits) {
  __hip_atomic_fetch_or(P.err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A wait that gave up: latch the timeout, tell every workgroup to stop waiting, and let
// the first one record where it was (workgroup, expected tag, word offset from the start
// of the exchange buffers, tag found there).
__device__ __forceinline__ void raise_timeout(const Params& P, const unsigned long long* where, uint32_t tag, uint32_t seen) {
  raise_error(P, DEV_ERR_TIMEOUT);
  __hip_atomic_store(P.abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(P.err + 3, &expected, 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    P.err[4] = blockIdx.x;
    P.err[5] = tag;
    P.err[6] = (uint32_t)(where - P.xq);
    P.err[7] = seen;
  }
}

// Loads per lane per poll round for an exchange of at most N words polled by NP waves: at
// most 8.
template <int N, int NP = 1, int CAP = 8>
struct Kp : std::integral_constant<int, (N + 64 * NP - 1) / (64 * NP) < CAP ? (N + 64 * NP - 1) / (64 * NP) : CAP> {};


// Gather words src[0..n) that other workgroups publish, waiting until each carries `tag`,
// into dst[0..n) (LDS).  Words [own0, own1) are this workgroup's own: the caller writes
// them to dst itself and they are not read back.  The words go in blocks of 64*KP; NPART
// waves may share a gather, wave `part` taking blocks part, part + NPART, ...
//
// Every round loads all KP words of a lane (indices clamped into the block), and
// `publish` (the caller's own stores, issued after the first round) stores
// unconditionally, so the number of memory operations between a round and its use is
// fixed and the wait before the first round does not cover the stores.  A new round is
// issued only after the previous one was consumed: a round still in flight when the
// gather completes would make the next reuse of its registers wait for it.  Returns
// false if the wait gave up (spin limit, or another workgroup's abort).
template <int KP, int NPART, class F>
__device__ __forceinline__ bool exchange(const u64* src, int n, uint32_t tag, float* dst, int own0, int own1, F&& publish,
                                         int lane, const Params& P, uint32_t& rounds, unsigned long long& first_round,
                                         int part) {
  static_assert(KP >= 1 && KP <= 16, "words per lane per round");
  bool published = false;
  for (int base = part * 64 * KP; base < n; base += NPART * 64 * KP) {
    const int cnt = min(n - base, 64 * KP);
    // need[k]: word base + lane + 64k is still awaited by this lane.  Each round only
    // selects (no branch per word): a word whose tag matches keeps its value in a register
    // and drops out of `need`; the values go to dst once the whole block has arrived.
    bool need[KP], want[KP];
    float val[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int i = base + lane + 64 * k;
      want[k] = need[k] = lane + 64 * k < cnt && (i < own0 || i >= own1);
      val[k] = 0.f;
    }
    const u64* s0 = src + base;
    const int last = cnt - 1;
    u64 wa[KP];
    auto issue = [&](u64(&w)[KP]) {
#pragma unroll
      for (int k = 0; k < KP; ++k) w[k] = ld_coh(s0 + min(lane + 64 * k, last));
    };
    auto absorb = [&](const u64(&w)[KP]) -> bool {
      bool left = false;
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const bool hit = (uint32_t)(w[k] >> 32) == tag;
        val[k] = hit ? __uint_as_float((uint32_t)w[k]) : val[k];
        need[k] = need[k] && !hit;
        left = left || need[k];
      }
      if (rounds++ == 0) first_round = wall_clock64();
      return !__any(left);
    };
    auto give_up = [&](const u64(&w)[KP]) {
      int k0 = -1;  // the first word still behind (selected without indexing w at run time)
      uint32_t seen = 0;
#pragma unroll
      for (int k = KP - 1; k >= 0; --k)
        if (need[k]) { k0 = k; seen = (uint32_t)(w[k] >> 32); }
      if (k0 >= 0) raise_timeout(P, s0 + lane + 64 * k0, tag, seen);
    };
    issue(wa);
    if (!published) {
      publish();
      published = true;
    }
    uint32_t it = 0;
    while (true) {
      if (absorb(wa)) break;
      if (++it >= P.spin_limit) {
        give_up(wa);
        return false;
      }
      if ((it & 127) == 0 && ld_coh32(P.abort_flag)) return false;
      issue(wa);
    }
#pragma unroll
    for (int k = 0; k < KP; ++k)
      if (want[k]) dst[base + lane + 64 * k] = val[k];
  }
  if (!published) publish();
  return true;
}

// ------------------------------------------------------------------ bf16 GEMV with split inputs
// An fp32 input v is carried as two bf16 values, hi = bf16(v) and lo = bf16(v - hi)
// (rounded to nearest even), so hi + lo keeps 16 significant bits; a weight pair times an
// input pair is then one packed dot-product instruction (bf16 products, fp32 sum), two per
// weight pair for hi and lo instead of a conversion and a multiply-add per weight.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// 8 consecutive inputs -> hi and lo chunks
__device__ __forceinline__ void split8(const float* v, u4& hi, u4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = v[2 * e], b = v[2 * e + 1];
    h[e] = pack_bf16(a, b);
    l[e] = pack_bf16(a - bf16lo(h[e]), b - bf16hi(h[e]));
  }
  hi = u4{h[0], h[1], h[2], h[3]};
  lo = u4{l[0], l[1], l[2], l[3]};
}
// (through a copy: a bit cast applied directly to a vector element has been seen to read
// element 0 instead)
__device__ __forceinline__ bf16x2 as_bf2(uint32_t u) {
  bf16x2 r;
  __builtin_memcpy(&r, &u, 4);
  return r;
}
__device__ __forceinline__ float dot2(uint32_t w, uint32_t a, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w), as_bf2(a), acc, false);
}
__device__ __forceinline__ float dot8(const u4& w, const u4& hi, const u4& lo, float acc) {
  acc = dot2(w.x, hi.x, acc);
  acc = dot2(w.y, hi.y, acc);
  acc = dot2(w.z, hi.z, acc);
  acc = dot2(w.w, hi.w, acc);
  acc = dot2(w.x, lo.x, acc);
  acc = dot2(w.y, lo.y, acc);
  acc = dot2(w.z, lo.z, acc);
  acc = dot2(w.w, lo.w, acc);
  return acc;
}

__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ LDS DMA
// One 16-byte chunk per lane from global memory straight into LDS: lane i's chunk lands at
// lds + 16 i.  Issued through inline assembly so that the compiler neither waits for it at
// barriers nor before unrelated LDS reads; completion is awaited explicitly with
// wait_vmem<N>() by the issuing wave, before a barrier, where N counts the vector-memory
// instructions this wave issued after it.  M0 (the LDS base register) is restored.
__device__ __forceinline__ void lds_dma16(const void* g, const void* lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(g), "s"(l) : "memory");
}
// s_waitcnt vmcnt(0) as a builtin (expcnt and lgkmcnt fields at their maxima), so that the
// compiler's own wait insertion knows no vector-memory load is outstanding after it.
__device__ __forceinline__ void vmem_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Worker waves 0..3 issue every weight copy of the LDS-tile bodies; waves 4..6 never have a


// Wait until at most c vector-memory instructions of this wave are pending (c wave-uniform).
template <int... I>
__device__ __forceinline__ void wait_vmem_table(int c, std::integer_sequence<int, I...>) {
  ((c == I ? (wait_vmem<I>(), 0) : 0), ...);
}
__device__ __forceinline__ void wait_vmem_rt(int c) {
  wait_vmem_table(min(c, 63), std::make_integer_sequence<int, 64>{});
}

}  // namespace mk
