// Small kernels beside the persistent one: the talker's input-row sum, the widening of
// gains to float32, and the self-tests of the LDS DMA copy and of the tagged-word
// exchange (the decode kernel's own primitives, from mk_device.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_device.h"
#include "mk_internal.h"

namespace mk {

// ------------------------------------------------------------------ small kernels
// Self-test of the LDS DMA primitive: the seven worker waves copy n chunks of src into LDS
// at byte offset off, wait for their copies, and every thread copies LDS back to dst.
// Exchange stress test of the tagged-word protocol every hop uses: `iters` rounds in
// which each workgroup publishes 64 words (tag tag0 + k, value a function of the
// workgroup, the round and the word) into its slot of buffer k & 1, then gathers all
// grid x 64 words of the round with `exchange`, the control wave and the seven worker
// waves taking blocks in turn as in the decode gathers.  Every gathered word is
// compared with the value its writer stored; bad[0] counts mismatches (a stale or torn
// word whose tag matched), bad[1] the workgroups whose wait gave up.  Two buffers
// suffice: a workgroup publishes round k + 1 only after it has read all of round k.
__device__ __forceinline__ float stress_value(int b, int k, int i) {
  return (float)((b * 977 + k * 131 + i * 7) & 0xffffff);  // exact in float32
}

// One round of the stress test for workgroup b: publish its 64 words (slot [own0, own0 +
// 64) of buf; LOCAL: with st_local) and gather the n words of buf into got.
template <int N, bool LOCAL>
__device__ __forceinline__ bool stress_round(const Params& P, u64* buf, int n, int own0, float* got, int k, int b,
                                             int wave, int lane, bool plain, uint32_t& rounds,
                                             unsigned long long& first_round) {
  constexpr int KP = Kp<N, kWorkerWaves + 1>::value;
  const uint32_t tag = P.tag0 + 1 + (uint32_t)k;
  bool ok;
  if (wave == 0) {
    ok = exchange<KP, kWorkerWaves + 1>(
        buf, n, tag, got, own0, own0 + 64,
        [&]() {
          const float v = stress_value(b, k, lane);
          if (LOCAL) st_local(buf + own0 + lane, v, tag, plain);
          else st_tag(buf + own0 + lane, v, tag);
          got[own0 + lane] = v;
        },
        lane, P, rounds, first_round, 0);
  } else {
    ok = exchange<KP, kWorkerWaves + 1>(buf, n, tag, got, own0, own0 + 64, []() {}, lane, P, rounds, first_round,
                                        wave);
  }
  return ok;
}

// iters rounds over the whole grid.  local == 0: all to all, every word written through to
// the device coherence point.  local != 0: each workgroup exchanges only with the 32 of
// its XCD (b % 8), and, when every workgroup sits on XCD b % 8 (checked first, as the
// decode kernel does), with plain stores that stay in that XCD's L2, the decode kernel's
// local hops; place: kGrid words for the placement check.  bad: [0] mismatched words,
// [1] workgroups whose wait gave up, [2] 1 if the plain stores were used.
__global__ void __launch_bounds__(kThreads) xchg_stress_kernel(Params P, u64* words, u64* place, int iters, int local,
                                                               uint32_t* bad) {
  constexpr int W = 64, N = kGrid * W, NL = kPerXcd * W;
  __shared__ float got[N];
  __shared__ int stop;
  const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = b % kXcds, r = b / kXcds;
  if (threadIdx.x == 0) stop = 0;
  __syncthreads();
  uint32_t rounds = 0;
  unsigned long long first_round = 0;
  bool plain = false;
  if (local) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    bool ok = true;
    if (wave == 0) {
      ok = exchange<Kp<kGrid>::value, 1>(
          place, kGrid, P.tag0, got, b, b + 1,
          [&]() {
            if (lane == 0) {
              st_tag(place + b, __uint_as_float(xcc & 0xfu), P.tag0);
              got[b] = __uint_as_float(xcc & 0xfu);
            }
          },
          lane, P, rounds, first_round, 0);
      if (!ok) stop = 1;
    }
    __syncthreads();
    bool on = true;
    for (int i = lane; i < kGrid; i += 64) on &= __float_as_uint(got[i]) == (uint32_t)(i % kXcds);
    plain = !stop && __all(on);
    __syncthreads();
  }
  for (int k = 0; k < iters && !stop; ++k) {
    u64* buf = words + (size_t)(k & 1) * N;
    bool ok;
    if (local)
      ok = stress_round<NL, true>(P, buf + g * NL, NL, r * W, got, k, b, wave, lane, plain, rounds, first_round);
    else
      ok = stress_round<N, false>(P, buf, N, b * W, got, k, b, wave, lane, false, rounds, first_round);
    if (!ok) stop = 1;
    __syncthreads();
    if (stop) break;
    uint32_t miss = 0;
    const int n = local ? NL : N;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int writer = local ? (i / W) * kXcds + g : i / W;
      miss += got[i] != stress_value(writer, k, i % W);
    }
    if (miss) atomicAdd(bad, miss);
    __syncthreads();
  }
  if (stop && threadIdx.x == 0) atomicAdd(bad + 1, 1u);
  if (b == 0 && threadIdx.x == 0 && plain) atomicAdd(bad + 2, 1u);
}

__global__ void __launch_bounds__(kThreads) lds_dma_selftest_kernel(const u4* src, u4* dst, int n, int off) {
  __shared__ __align__(16) u4 buf[144 * 1024 / 16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  u4* base = buf + off / 16;
  if (wave < kWorkerWaves) {
    const int ni = (n + 63) / 64;
    for (int i = wave; i < ni; i += kWorkerWaves) lds_dma16(src + min(i * 64 + lane, n - 1), base + i * 64);
    wait_vmem<0>();
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = base[i];
}

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

int launch_embed_sum(const void* codebooks, int n_cb, int cb_size, const void* text, int text_vocab, int hidden,
                     int bf16, const int32_t* ids, int n, float* rows, int32_t* bad, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(embed_sum_kernel, dim3(n), dim3(256), 0, (hipStream_t)stream, codebooks, n_cb, cb_size, text,
                     text_vocab, hidden, bf16, ids, rows, bad);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_exchange_stress(const Params& p, unsigned long long* words, unsigned long long* place, int iters, int local,
                           uint32_t* bad, void* stream) {
  Params pp = p;
  u64* w = words;
  u64* pl = place;
  void* args[] = {&pp, &w, &pl, &iters, &local, &bad};
  hipError_t e = hipLaunchCooperativeKernel((const void*)xchg_stress_kernel, dim3(kGrid), dim3(kThreads), args, 0,
                                            (hipStream_t)stream);
  return e == hipSuccess ? 0 : -1;
}

int launch_lds_dma_selftest(const void* src, void* dst, int n_chunks, int offset_bytes, void* stream) {
  hipLaunchKernelGGL(lds_dma_selftest_kernel, dim3(1), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u4*)src, (u4*)dst, n_chunks, offset_bytes);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_widen(const void* src, float* dst, int n, int bf16, void* stream) {
  hipLaunchKernelGGL(widen_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, src, dst, n, bf16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mk
