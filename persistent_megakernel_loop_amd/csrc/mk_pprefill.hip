// Batched prompt prefill as one persistent launch per chunk of up to 64 positions.
//
// The kernel-chain form (mk_prefill.hip) runs nine dependent kernels per layer, and a
// short prompt spends most of its time in their launches and ramps, not in the weight
// pass.  Here one cooperative launch of 256 workgroups stays resident for every layer of
// a chunk, and the phases of a layer hand their results over the way the decode kernel's
// do, without kernel boundaries: the producer writes its block, waits until its stores
// have completed, then raises a tagged flag word; the consumer polls the flags of the
// producers it needs and reads their blocks with device-coherent loads.
//
// The work is split as in the decode kernel (KV group g and MLP slice g on XCD g; the
// residual owned by columns and kept once per XCD), with every product on the matrix
// cores over the chunk's positions (16x16x32 bf16 MFMA; activations split into bf16 high
// and low parts, two products per tile, as in the chain):
//
//   q/k/v      group g's 512 rows on XCD g, 16 rows per workgroup, all hidden columns
//   attention  one workgroup per (group, position): q/k RMSNorm and the rotary of the
//              multi-section streams, the cache rows of its position, then causal
//              attention over the cached keys and the chunk's own
//   O          XCD g multiplies its group's 256 attention columns into 32 hidden rows per
//              workgroup: one partial per XCD
//   residual   workgroup j of every XCD owns hidden columns 32j..32j+31 and adds the 8
//              partials in XCD order, so every XCD holds the same residual
//   gate/up    slice g on XCD g: 12 gate rows and the matching 12 up rows per workgroup,
//              then the SwiGLU of those 12 columns
//   down       XCD g multiplies its slice's 384 columns into 32 hidden rows per workgroup
//   residual   as above, then the next layer's input norm
//
// That is seven hand-overs per layer, two of them across XCDs (the partials).  Each norm
// is folded as in the chain: a product's operand is gains * x, and its consumer scales by
// 1/rms from sums of squares that the owners publish with the operand.
//
// Memory ordering.  Inside an XCD (placement checked at launch, as the decode kernel
// does) blocks and flags are plain stores, which stay in the XCD's L2, where the readers'
// device-coherent loads find them.  Across XCDs, or if the placement check fails, blocks
// and flags are written through at device scope.  A producer raises its flag only after
// all its waves have waited for their stores (vmcnt 0) and met at a barrier; consumers
// read blocks only after their flags carry the current tag.  Tags are unique per launch
// and phase, so flag words never need clearing between launches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_device.h"
#include "mk_internal.h"
#include "mk_prefill.h"

namespace mk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 128, kQpg = 2, kH = 1024, kI = 3 * kH;
constexpr int kCw = kH / kPerXcd;              // 32 residual columns per owner
constexpr int kIx = kI / kXcds;                // 384 MLP columns per XCD
constexpr int kHalf = kI / (kXcds * kPerXcd);  // 12 gate rows (and 12 up rows) per workgroup
constexpr int kQRows = (kQpg + 2) * kD;        // 512 q/k/v rows per group
constexpr int kPpThreads = 512;
constexpr int kKRow = kD + 8;                  // LDS key row stride (u16): spreads the lanes' rows over banks
enum : int { KQ = 0, KA = 1, KO = 2, KR1 = 3, KG = 4, KD = 5, KR2 = 6, KPLACE = 7 };
static_assert(KPLACE < kPpKinds, "flag kinds");

struct PpK {
  PfArgs A;
  PpBufs B;
  const uint8_t* layers;
  LayerLayout lay;
  uint32_t tag0;
  uint32_t spin_limit;
  uint32_t* abort_flag;
  unsigned long long* dbg;  // phase timeline [grid][L + 1][kPpKinds][2], or NULL
};

__device__ __forceinline__ uint32_t pp_tag(uint32_t tag0, int l, int kind) {
  return tag0 + (uint32_t)(l + 1) * (uint32_t)kPpKinds + (uint32_t)kind;
}

// A device buffer addressed through a buffer resource: loads are device-coherent (they
// bypass the CU's L1), stores are plain or written through at device scope, and an
// offset past `bytes` reads 0 and drops the store instead of faulting.
struct Buf {
  __amdgpu_buffer_rsrc_t r;
  __device__ Buf(const void* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000)) {}
  __device__ u4 ld16(uint32_t off) const { return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 16); }
  __device__ uint32_t ld4(uint32_t off) const { return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 16); }
  __device__ void st16(uint32_t off, u4 v, bool plain) const {
    if (plain) __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 16);
  }
  __device__ void st4(uint32_t off, uint32_t v, bool plain) const {
    if (plain) __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 16);
  }
  __device__ void st2(uint32_t off, uint16_t v, bool plain) const {
    if (plain) __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, 16);
  }
};

__device__ __forceinline__ bf16x8 as_bf8(u4 v) { return __builtin_bit_cast(bf16x8, v); }
// A phase's weight pointer, made opaque where the phase starts: its loads cannot be
// hoisted into earlier phases, where their registers would stay live across the waits.
template <class T>
__device__ __forceinline__ T opaque(T v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ uint16_t to_bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float from_bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ void pp_raise(const PpK& k, uint32_t bits) {
  __hip_atomic_fetch_or(k.A.err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A wait that gave up: latch the timeout, stop every other wait, and record the first
// one (workgroup, expected tag, flag index with bit 31 set to tell it from the decode
// kernel's word offsets, tag found).
__device__ void pp_timeout(const PpK& k, uint32_t where, uint32_t tag, uint32_t seen) {
  pp_raise(k, DEV_ERR_TIMEOUT);
  __hip_atomic_store(k.abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(k.A.err + 3, &expected, 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    k.A.err[4] = blockIdx.x;
    k.A.err[5] = tag;
    k.A.err[6] = where | 0x80000000u;
    k.A.err[7] = seen;
  }
}

// Wave 0 polls the flags of n workgroups (flag index base + i * step, i < n <= 64) until
// each carries `tag`; then the workgroup meets at a barrier.  Returns false on every
// thread if the wait gave up (spin limit) or another workgroup's wait did.
// Timeline record of hand-over `kind` produced in layer pl (-1: the input rows):
// e = 0 when this workgroup's wait for it completed, e = 1 when it raised its own flag.
__device__ __forceinline__ void stamp(const PpK& k, int pl, int kind, int e) {
  if (k.dbg) k.dbg[(((size_t)blockIdx.x * (k.A.L + 1) + pl + 1) * kPpKinds + kind) * 2 + e] = wall_clock64();
}

__device__ bool wg_wait(const PpK& k, int tid, int kind, int base, int step, int n, uint32_t tag, int* stop, int pl) {
  if (tid < 64) {
    const int lane = tid;
    const uint32_t idx = (uint32_t)(kind * kGrid + base + min(lane, n - 1) * step);
    const u64* f = k.B.flags + idx;
    uint32_t it = 0;
    bool ok = false;
    while (true) {
      const uint32_t seen = (uint32_t)(ld_coh(f) >> 32);
      ok = seen == tag;
      if (__all(ok)) break;
      if (++it >= k.spin_limit) {
        if (!ok) pp_timeout(k, idx, tag, seen);
        break;
      }
      if ((it & 127) == 0 && ld_coh32(k.abort_flag)) break;
    }
    const bool all_ok = __all(ok);
    if (lane == 0) *stop = all_ok ? 0 : 1;
  }
  __syncthreads();
  if (tid == 0) stamp(k, pl, kind, 0);
  return *stop == 0;
}

// Every wave waits for its own stores, the workgroup meets, and thread 0 raises the flag.
__device__ __forceinline__ void wg_publish(const PpK& k, int kind, uint32_t tag, bool plain, int pl) {
  vmem_drain();
  __syncthreads();
  if (threadIdx.x == 0) {
    st_local(k.B.flags + kind * kGrid + blockIdx.x, 0.f, tag, plain);
    stamp(k, pl, kind, 1);
  }
}

// acc[nt] += A (16 rows x 64 columns) * B (the same 64 columns x 16 positions of tile nt).
// Lane (q, i) = (lane / 16, lane % 16) holds row i of A and position i of B over columns
// 16q + 8hf .. +7 for hf = 0, 1, so both operands of an MFMA cover the same 32 columns
// whatever order the instruction pairs them in; B comes as high and low parts.
template <int NT>
__device__ __forceinline__ void mfma_step(const bf16x8 (&a)[2], const bf16x8 (&bh)[NT][2], const bf16x8 (&bl)[NT][2],
                                          f4 (&acc)[NT]) {
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[hf], bh[nt][hf], acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[hf], bl[nt][hf], acc[nt], 0, 0, 0);
    }
}

// The split operand's 64-column step starting at 8-column chunk ch0: element (k, n) of a
// K-column operand sits at [(k / 8) * NPP + n][k % 8], high parts first, the low parts
// K * NPP elements further.
template <int NT>
__device__ __forceinline__ void load_b(const Buf& src, int K, int ch0, int lane, bf16x8 (&bh)[NT][2],
                                       bf16x8 (&bl)[NT][2]) {
  constexpr int NPP = 16 * NT;
  const int q = lane >> 4, i = lane & 15;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t off = (uint32_t)(((ch0 + 2 * q + hf) * NPP + 16 * nt + i) * 16);
      bh[nt][hf] = as_bf8(src.ld16(off));
      bl[nt][hf] = as_bf8(src.ld16(off + (uint32_t)(K * NPP * 2)));
    }
}

// Row `row` of a bf16 matrix with leading dimension ld, columns k0 + 16q + 8hf .. +7.
__device__ __forceinline__ void load_a(const uint16_t* w, size_t row, int ld, int k0, int lane, bf16x8 (&a)[2]) {
  const uint16_t* p = w + row * (size_t)ld + k0 + 16 * (lane >> 4);
  a[0] = *reinterpret_cast<const bf16x8*>(p);
  a[1] = *reinterpret_cast<const bf16x8*>(p + 8);
}

// 1/rms of every position from the 32 owners' sums of squares (in owner order).
template <int NPP>
__device__ __forceinline__ void rms_of(const Buf& ss, float eps, float* rs, int tid) {
  const int n = tid;
  if (n < NPP) {
    float part[kPerXcd];
#pragma unroll
    for (int o = 0; o < kPerXcd; ++o) part[o] = __uint_as_float(ss.ld4((uint32_t)((o * NPP + n) * 4)));
    float s = 0.f;
#pragma unroll
    for (int o = 0; o < kPerXcd; ++o) s += part[o];
    rs[n] = rsqrtf(s / (float)kH + eps);
  }
}

// Owner j publishes its residual columns for a product: gains * x split into the
// operand layout, and the sums of squares of x over its columns per position.
// The 8 gains of the columns thread tid publishes (they do not depend on the position),
// loaded ahead of the phase's other memory round trips.
__device__ __forceinline__ void load_gains(const float* g, int j, int tid, float (&g8)[8]) {
  const int col = kCw * j + 8 * (tid % (kCw / 8));
  const float4 a = *reinterpret_cast<const float4*>(g + col), b = *reinterpret_cast<const float4*>(g + col + 4);
  g8[0] = a.x; g8[1] = a.y; g8[2] = a.z; g8[3] = a.w; g8[4] = b.x; g8[5] = b.y; g8[6] = b.z; g8[7] = b.w;
}

template <int NPP>
__device__ __forceinline__ void publish_residual(const float (&xres)[NPP][kCw], const float (&g8)[8], int j,
                                                 const Buf& dst, const Buf& ss, bool plain, int tid) {
  const int t = tid;
  if (t < NPP * (kCw / 8)) {
    const int n = t / (kCw / 8), c8 = t % (kCw / 8), col = kCw * j + 8 * c8;
    float v[8], gv[8], sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = xres[n][8 * c8 + e];
      gv[e] = g8[e] * v[e];
      sq = fmaf(v[e], v[e], sq);
    }
    u4 hi, lo;
    split8(gv, hi, lo);
    const uint32_t off = (uint32_t)((((col >> 3) * NPP) + n) * 16);
    dst.st16(off, hi, plain);
    dst.st16(off + (uint32_t)(kH * NPP * 2), lo, plain);
    sq = group_sum<kCw / 8>(sq);
    if (c8 == kCw / 8 - 1) ss.st4((uint32_t)((j * NPP + n) * 4), __float_as_uint(sq), plain);
  }
}

// The 8 XCDs' partials of owner j's columns (in XCD order) added to its residual.
template <int NPP>
__device__ __forceinline__ void add_partials(float (&xres)[NPP][kCw], const Buf& part, int j, int tid) {
  const int t = tid;
  if (t < NPP * (kCw / 4)) {
    const int n = t / (kCw / 4), c4 = t % (kCw / 4);
    u4 v[kXcds];
#pragma unroll
    for (int g = 0; g < kXcds; ++g) v[g] = part.ld16((uint32_t)((((g * kPerXcd + j) * NPP + n) * kCw + 4 * c4) * 4));
    float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < kXcds; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] += __uint_as_float(v[g][e]);
#pragma unroll
    for (int e = 0; e < 4; ++e) xres[n][4 * c4 + e] += y[e];
  }
}

// The rotary table of the chunk's positions: pair i (elements i and i + 64) of position
// n at the position stream its section reads (a stream value outside the table reads
// row 0, as it is flagged), gathered into LDS once per launch.
template <int NPP>
__device__ __forceinline__ void rope_table(const PfArgs& A, float (&rc)[NPP][kD / 2], float (&rsn)[NPP][kD / 2]) {
  for (int u = threadIdx.x; u < NPP * (kD / 2); u += kPpThreads) {
    const int n = u / (kD / 2), i = u % (kD / 2);
    float c = 1.f, sn = 0.f;
    if (n < A.m) {
      const int sct = i < A.sec_end0 ? 0 : (i < A.sec_end1 ? 1 : 2);
      int ps = A.pos3 ? A.pos3[n * 3 + sct] : A.pos0 + n;
      ps = (ps < 0 || ps >= A.rope_positions) ? 0 : ps;
      c = A.rope_cos[(size_t)ps * (kD / 2) + i];
      sn = A.rope_sin[(size_t)ps * (kD / 2) + i];
    }
    rc[n][i] = c;
    rsn[n][i] = sn;
  }
}

// RMSNorm over the head (gains gn) and the rotary of pair i, for a lane holding elements
// i and i + 64 of the head; returns them in a0, a1.
__device__ __forceinline__ void norm_rotate(const float* gn, float eps, float c, float sn, int i, float& a0, float& a1) {
  const float sq = wave_sum(fmaf(a1, a1, a0 * a0));
  const float r = rsqrtf(sq / (float)kD + eps);
  const float n0 = gn[i] * (a0 * r), n1 = gn[i + 64] * (a1 * r);
  a0 = n0 * c - n1 * sn;
  a1 = n1 * c + n0 * sn;
}

// LDS of the attention phase.
struct AttLds {
  float qs[2][kQpg][kD];              // the workgroup's (up to two) positions' rotated, scaled queries
  uint16_t kl[kPrefillChunk][kKRow];  // the chunk's keys after norm and rotary, bf16
  uint16_t vl[kPrefillChunk][kD];     // the chunk's values, bf16
  float pw[8][kQpg][64];              // a block's softmax weights, per wave
  float sl[kQpg][64];                 // scores of a one-block context
  float mw[8][kQpg], lw[8][kQpg];
  float aw[8][kQpg][kD];
};

// Scores of key row tt against both query heads of slot s: the row from the cache below
// pos0, else the chunk's own from LDS.  The row is read in two halves of 64 dims (a
// half's loads all in flight at once), and the queries from LDS (one broadcast read per
// 4 dims) inside the loop: an offset the compiler cannot see through keeps it from
// holding all 256 in registers.
__device__ __forceinline__ void score_row(const PfArgs& A, const AttLds& S, int s, size_t cbase, int tt, int pos0,
                                          float (&sc)[kQpg]) {
  sc[0] = sc[1] = 0.f;
  int qo = 0;
  asm volatile("" : "+v"(qo));
  const float* qsp = &S.qs[s][0][0] + qo;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint4 kr[kD / 16];
    if (tt < pos0) {
#pragma unroll
      for (int j8 = 0; j8 < kD / 16; ++j8)
        kr[j8] = *reinterpret_cast<const uint4*>(A.kcache + cbase + (size_t)tt * kD + 64 * half + 8 * j8);
    } else {
#pragma unroll
      for (int j8 = 0; j8 < kD / 16; ++j8)
        kr[j8] = *reinterpret_cast<const uint4*>(&S.kl[tt - pos0][64 * half + 8 * j8]);
    }
#pragma unroll
    for (int j8 = 0; j8 < kD / 16; ++j8) {
      const uint32_t wd[4] = {kr[j8].x, kr[j8].y, kr[j8].z, kr[j8].w};
      const int d0 = 64 * half + 8 * j8;
#pragma unroll
      for (int h = 0; h < kQpg; ++h) {
        const float4 qa = *reinterpret_cast<const float4*>(qsp + h * kD + d0);
        const float4 qb = *reinterpret_cast<const float4*>(qsp + h * kD + d0 + 4);
        const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[h] = fmaf(qv[2 * e], bf16lo(wd[e]), sc[h]);
          sc[h] = fmaf(qv[2 * e + 1], bf16hi(wd[e]), sc[h]);
        }
      }
      if (j8 & 1) __builtin_amdgcn_sched_barrier(0);  // at most 4 query reads in flight per head
    }
  }
}

// Head h's attention output for position n (dims 2 lane, 2 lane + 1), split into the O
// product's operand.
template <int NPP>
__device__ __forceinline__ void store_att(const Buf& at, bool plain, int n, int h, int lane, float o0, float o1) {
  const uint16_t h0 = to_bf(o0), h1 = to_bf(o1);
  const uint16_t l0 = to_bf(o0 - from_bf(h0)), l1 = to_bf(o1 - from_bf(h1));
  const int c = h * kD + 2 * lane;
  const uint32_t off = (uint32_t)((((c >> 3) * NPP + n) * 8 + (c & 7)) * 2);
  at.st4(off, (uint32_t)h0 | ((uint32_t)h1 << 16), plain);
  at.st4(off + (uint32_t)(kQpg * kD * NPP * 2), (uint32_t)l0 | ((uint32_t)l1 << 16), plain);
}

// Causal attention of position n (query slot s of the workgroup) for group g over keys
// 0..pos0+n: keys below pos0 from the cache, the chunk's own from LDS.  Wave w takes the
// 64-key blocks w, w + 8, ...: lane j scores key j against both query heads, the block's
// softmax weights go through LDS, and each lane accumulates value dims 2j, 2j + 1.  The
// waves' maxima, sums and outputs are merged in wave order; the output goes out split
// into the O product's operand.
template <int NPP>
__device__ void attend(const PpK& k, AttLds& S, int l, int g, int n, int s, const Buf& at, bool plain, int tid) {
  const PfArgs& A = k.A;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int p = A.pos0 + n, nkeys = p + 1, pos0 = A.pos0;
  const size_t cbase = ((size_t)l * kXcds + g) * A.max_seq * kD;
  // A context of one block (up to 64 keys): every wave scores 8 keys (8 lanes per key,
  // 16 dims per lane, summed over the 8 lanes), wave 0 normalises the weights, and all
  // waves share the value sum, 8 rows each.  Longer: every wave runs its own blocks with
  // a running maximum and sum, merged across waves at the end.
  const bool one_block = nkeys <= 64;
  if (one_block) {
    const int kk = lane >> 3, d16 = lane & 7, t = 8 * w + kk;
    const bool valid = t < nkeys;
    const int tt = valid ? t : p;
    uint4 kr[2];
    if (tt < pos0) {
      kr[0] = *reinterpret_cast<const uint4*>(A.kcache + cbase + (size_t)tt * kD + 16 * d16);
      kr[1] = *reinterpret_cast<const uint4*>(A.kcache + cbase + (size_t)tt * kD + 16 * d16 + 8);
    } else {
      kr[0] = *reinterpret_cast<const uint4*>(&S.kl[tt - pos0][16 * d16]);
      kr[1] = *reinterpret_cast<const uint4*>(&S.kl[tt - pos0][16 * d16 + 8]);
    }
#pragma unroll
    for (int h = 0; h < kQpg; ++h) {
      float sc = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float4 qa = *reinterpret_cast<const float4*>(&S.qs[s][h][16 * d16 + 8 * c]);
        const float4 qb = *reinterpret_cast<const float4*>(&S.qs[s][h][16 * d16 + 8 * c + 4]);
        const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
        const uint32_t wd[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc = fmaf(qv[2 * e], bf16lo(wd[e]), sc);
          sc = fmaf(qv[2 * e + 1], bf16hi(wd[e]), sc);
        }
      }
      sc = group_sum<8>(sc);
      if (d16 == 7) S.sl[h][t] = valid ? sc : -INFINITY;
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int h = 0; h < kQpg; ++h) {
        const bool vl = lane < nkeys;
        const float sv = vl ? S.sl[h][lane] : -INFINITY;
        const float mx = wave_max(sv);
        const float pr = vl ? __expf(sv - mx) : 0.f;
        S.pw[0][h][lane] = pr / wave_sum(pr);
      }
    }
    __syncthreads();
    float acc[kQpg][2] = {{0.f, 0.f}, {0.f, 0.f}};
    if (8 * w < nkeys) {
      uint32_t vv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int row = min(8 * w + u, nkeys - 1);
        vv[u] = row < pos0 ? *reinterpret_cast<const uint32_t*>(A.vcache + cbase + (size_t)row * kD + 2 * lane)
                           : *reinterpret_cast<const uint32_t*>(&S.vl[row - pos0][2 * lane]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int h = 0; h < kQpg; ++h) {
          const float pu = 8 * w + u < nkeys ? S.pw[0][h][8 * w + u] : 0.f;
          acc[h][0] = fmaf(pu, bf16lo(vv[u]), acc[h][0]);
          acc[h][1] = fmaf(pu, bf16hi(vv[u]), acc[h][1]);
        }
    }
#pragma unroll
    for (int h = 0; h < kQpg; ++h) {
      S.aw[w][h][2 * lane] = acc[h][0];
      S.aw[w][h][2 * lane + 1] = acc[h][1];
    }
    __syncthreads();
    if (w < kQpg) {
      const int h = w;
      float o0 = 0.f, o1 = 0.f;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        o0 += S.aw[v][h][2 * lane];
        o1 += S.aw[v][h][2 * lane + 1];
      }
      store_att<NPP>(at, plain, n, h, lane, o0, o1);
    }
    __syncthreads();
    return;
  }
  float M[kQpg], Ls[kQpg], acc[kQpg][2];
#pragma unroll
  for (int h = 0; h < kQpg; ++h) { M[h] = -INFINITY; Ls[h] = 0.f; acc[h][0] = acc[h][1] = 0.f; }
#pragma nounroll
  for (int kb = w; kb * 64 < nkeys; kb += 8) {
    const int t = kb * 64 + lane;
    const bool valid = t < nkeys;
    const int tt = valid ? t : p;
    float sc[kQpg];
    score_row(A, S, s, cbase, tt, pos0, sc);
#pragma unroll
    for (int h = 0; h < kQpg; ++h) {
      const float sv = valid ? sc[h] : -INFINITY;
      const float mn = fmaxf(M[h], wave_max(sv));  // finite: key kb*64 is valid
      const float corr = __expf(M[h] - mn);        // 0 while M is still -inf
      const float pr = valid ? __expf(sv - mn) : 0.f;
      Ls[h] = Ls[h] * corr + wave_sum(pr);
      acc[h][0] *= corr;
      acc[h][1] *= corr;
      M[h] = mn;
      S.pw[w][h][lane] = pr;
    }
    __builtin_amdgcn_wave_barrier();
    const int nb = min(64, nkeys - kb * 64);
#pragma nounroll
    for (int e0 = 0; e0 < nb; e0 += 8) {
      uint32_t vv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int row = kb * 64 + min(e0 + u, nb - 1);
        vv[u] = row < pos0 ? *reinterpret_cast<const uint32_t*>(A.vcache + cbase + (size_t)row * kD + 2 * lane)
                           : *reinterpret_cast<const uint32_t*>(&S.vl[row - pos0][2 * lane]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int h = 0; h < kQpg; ++h) {
          const float pu = e0 + u < nb ? S.pw[w][h][e0 + u] : 0.f;
          acc[h][0] = fmaf(pu, bf16lo(vv[u]), acc[h][0]);
          acc[h][1] = fmaf(pu, bf16hi(vv[u]), acc[h][1]);
        }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int h = 0; h < kQpg; ++h) {
    if (lane == 0) { S.mw[w][h] = M[h]; S.lw[w][h] = Ls[h]; }
    S.aw[w][h][2 * lane] = acc[h][0];
    S.aw[w][h][2 * lane + 1] = acc[h][1];
  }
  __syncthreads();
  if (w < kQpg) {
    const int h = w;
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 8; ++v) mx = fmaxf(mx, S.mw[v][h]);
    float f[8], lsum = 0.f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      f[v] = S.mw[v][h] == -INFINITY ? 0.f : __expf(S.mw[v][h] - mx);
      lsum = fmaf(f[v], S.lw[v][h], lsum);
    }
    const float inv = 1.f / lsum;
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      o0 = fmaf(f[v], S.aw[v][h][2 * lane], o0);
      o1 = fmaf(f[v], S.aw[v][h][2 * lane + 1], o1);
    }
    store_att<NPP>(at, plain, n, h, lane, o0 * inv, o1 * inv);
  }
  __syncthreads();  // the LDS partials are reused by the workgroup's next position
}

// The weight tiles of each product for wave w, from layer l's tiles.  (The layer pointer
// goes through opaque() so that the compiler keeps each load where it is written.)
__device__ __forceinline__ const uint16_t* layer_tiles(const PpK& k, int l, size_t off) {
  return opaque(reinterpret_cast<const uint16_t*>(k.layers + (size_t)l * k.lay.stride + off));
}
// q/k/v: rows 16j .. 16j + 15 of group x, columns 128w .. 128w + 127 in two steps.
__device__ __forceinline__ void ld_q(const PpK& k, int l, int x, int j, int w, int lane, bf16x8 (&a)[2][2]) {
  const uint16_t* wq = layer_tiles(k, l, k.lay.qkv);
#pragma unroll
  for (int s = 0; s < 2; ++s) load_a(wq, (size_t)x * kQRows + 16 * j + (lane & 15), kH, 128 * w + 64 * s, lane, a[s]);
}
// O (waves 0..3): rows 32j .. 32j + 31 of KV block x as two row tiles, columns 64w .. +63:
// each operand step is read by one wave only.
__device__ __forceinline__ void ld_o(const PpK& k, int l, int x, int j, int w, int lane, bf16x8 (&a)[2][2]) {
  const uint16_t* wo = layer_tiles(k, l, k.lay.o) + (size_t)x * kH * (kQpg * kD);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) load_a(wo, (size_t)(kCw * j + 16 * rt + (lane & 15)), kQpg * kD, 64 * w, lane, a[rt]);
}
// gate/up: rows 24j .. 24j + 23 of slice x (two row tiles, the second half empty),
// columns 128w .. 128w + 127 in two steps.
__device__ __forceinline__ void ld_g(const PpK& k, int l, int x, int j, int w, int lane, bf16x8 (&a)[2][2][2]) {
  const uint16_t* wg = layer_tiles(k, l, k.lay.gu);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int rl = 16 * rt + (lane & 15);
      if (rl < 2 * kHalf) {
        load_a(wg, (size_t)x * 2 * kIx + 2 * kHalf * j + rl, kH, 128 * w + 64 * s, lane, a[rt][s]);
      } else {
        a[rt][s][0] = as_bf8(u4{0u, 0u, 0u, 0u});
        a[rt][s][1] = as_bf8(u4{0u, 0u, 0u, 0u});
      }
    }
}
// down (waves 0..5): rows 32j .. 32j + 31 of slice x as two row tiles, columns 64w .. +63
// of the slice's 384: each operand step is read by one wave only.
__device__ __forceinline__ void ld_d(const PpK& k, int l, int x, int j, int w, int lane, bf16x8 (&a)[2][2]) {
  const uint16_t* wd = layer_tiles(k, l, k.lay.down) + (size_t)x * kH * kIx;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) load_a(wd, (size_t)(kCw * j + 16 * rt + (lane & 15)), kIx, 64 * w, lane, a[rt]);
}

template <int NT>
__global__ __launch_bounds__(kPpThreads) void pp_kernel(PpK k) {
  constexpr int NPP = 16 * NT;
  constexpr size_t kRedBytes = (size_t)8 * 2 * NT * 64 * sizeof(f4);
  constexpr size_t kBig = kRedBytes > sizeof(AttLds) ? kRedBytes : sizeof(AttLds);
  __shared__ __align__(16) float xres[NPP][kCw];
  __shared__ __align__(16) float gu[NPP][2 * kHalf];
  __shared__ float rs[NPP];
  __shared__ float rc[NPP][kD / 2], rsn[NPP][kD / 2];  // the chunk's rotary table
  __shared__ int stop, placed_s;
  __shared__ __align__(16) u4 big[kBig / 16];
  f4* red = reinterpret_cast<f4*>(big);
  AttLds& S = *reinterpret_cast<AttLds*>(big);

  const PfArgs& A = k.A;
  const int b = blockIdx.x, x = b % kXcds, j = b / kXcds;
  const int m = A.m, L = A.L;

  // Region views of this XCD's replicas (sized for this chunk's NPP).
  const uint32_t xs_bytes = (uint32_t)(2 * kH * NPP * 2);
  const Buf xb(k.B.xb + (size_t)x * 2 * kH * NPP, xs_bytes);
  const Buf xp(k.B.xp + (size_t)x * 2 * kH * NPP, xs_bytes);
  const Buf ss(k.B.ss + (size_t)x * kPerXcd * NPP, (uint32_t)(kPerXcd * NPP * 4));
  const Buf ss2(k.B.ss2 + (size_t)x * kPerXcd * NPP, (uint32_t)(kPerXcd * NPP * 4));
  const Buf qr(k.B.qr + (size_t)x * NPP * kQRows, (uint32_t)(NPP * kQRows * 4));
  const Buf at(k.B.at + (size_t)x * 2 * kQpg * kD * NPP, (uint32_t)(2 * kQpg * kD * NPP * 2));
  const Buf hs(k.B.hs + (size_t)x * 2 * kIx * NPP, (uint32_t)(2 * kIx * NPP * 2));
  const Buf op(k.B.op, (uint32_t)(kXcds * kPerXcd * NPP * kCw * 4));
  const Buf dp(k.B.dp, (uint32_t)(kXcds * kPerXcd * NPP * kCw * 4));

  // ---------------------------------------------------------------- placement
  if (threadIdx.x == 0) stamp(k, -1, KPLACE, 0);
  if (threadIdx.x == 0) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    st_tag(k.B.flags + KPLACE * kGrid + b, __uint_as_float(xcc & 0xfu), pp_tag(k.tag0, -1, KPLACE));
  }
  rope_table<NPP>(A, rc, rsn);  // read after the barrier that ends the placement check
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint32_t tag = pp_tag(k.tag0, -1, KPLACE);
    const u64* f = k.B.flags + KPLACE * kGrid;
    uint32_t it = 0, seen[kGrid / 64];
    bool ok = false, done = false;
    while (true) {
      ok = true;
#pragma unroll
      for (int u = 0; u < kGrid / 64; ++u) {
        const u64 wd = ld_coh(f + lane + 64 * u);
        seen[u] = (uint32_t)wd;
        ok = ok && (uint32_t)(wd >> 32) == tag;
      }
      if (__all(ok)) { done = true; break; }
      if (++it >= k.spin_limit) {
        if (!ok) pp_timeout(k, (uint32_t)(KPLACE * kGrid + lane), tag, 0);
        break;
      }
      if ((it & 127) == 0 && ld_coh32(k.abort_flag)) break;
    }
    bool here = true;
#pragma unroll
    for (int u = 0; u < kGrid / 64; ++u) here = here && seen[u] == (uint32_t)((lane + 64 * u) % kXcds);
    const bool all_here = __all(here);
    if (lane == 0) {
      stop = done ? 0 : 1;
      placed_s = all_here ? 1 : 0;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) stamp(k, -1, KPLACE, 1);
  if (stop) return;
  const bool plain = placed_s != 0;  // XCD-local blocks and flags may stay in the XCD's L2

  // ---------------------------------------------------------------- input rows
  {
    const int t = threadIdx.x;
    if (b == 0) {
      for (int u = t; u < m * 3; u += kPpThreads) {
        const int n = u / 3, sct = u % 3;
        if (sct < A.n_sections) {
          const int v = A.pos3 ? A.pos3[n * 3 + sct] : A.pos0 + n;
          if (v < 0 || v >= A.rope_positions) pp_raise(k, DEV_ERR_POS);
        }
      }
    }
    if (t < NPP * (kCw / 8)) {
      const int n = t / (kCw / 8), c8 = t % (kCw / 8), col = kCw * j + 8 * c8;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (n < m) {
        int id = A.ids[n];
        if (id >= A.vocab || (id < 0 && A.rows == nullptr)) {  // flagged and read as id 0
          if (b == 0 && c8 == 0) pp_raise(k, DEV_ERR_ID);
          id = 0;
        }
        if (id >= 0) {
          const uint4 u = *reinterpret_cast<const uint4*>(A.embed + (size_t)id * kH + col);
          const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16lo(wd[e]);
            v[2 * e + 1] = bf16hi(wd[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = A.rows[(size_t)n * kH + col + e];
        }
        if (x == 0 && A.dbg_hidden)
#pragma unroll
          for (int e = 0; e < 8; ++e) A.dbg_hidden[(size_t)n * (L + 1) * kH + col + e] = v[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) xres[n][8 * c8 + e] = v[e];
    }
    float g8[8];
    load_gains(A.in_norm0, j, threadIdx.x, g8);
    __syncthreads();
    publish_residual<NPP>(xres, g8, j, xb, ss, plain, (int)threadIdx.x);
    wg_publish(k, KR2, pp_tag(k.tag0, -1, KR2), plain, -1);
  }
  // The products' weight tiles, loaded by every wave right before the phase's wait, so
  // that they arrive while it waits.  Two other placements were slower: loading them a
  // phase earlier put them ahead of the operand loads of the phase in between, in the
  // same in-order memory queue; and letting wave 0, which polls the flags, load its share
  // only after the poll exposed the whole load latency to its product.
  bf16x8 aQ[2][2], aO[2][2], aG[2][2][2], aD[2][2];

#pragma nounroll
  for (int l = 0; l < L; ++l) {
    // The thread index, made opaque once per layer: every lane- and wave-dependent offset
    // (and row test) is computed inside the layer instead of being hoisted out of the loop,
    // where all phases' offsets would stay live (in registers) at once.
    const int tid = opaque((int)threadIdx.x), lane = tid & 63, li = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint8_t* base = k.layers + (size_t)l * k.lay.stride;
    const float* G = reinterpret_cast<const float*>(base + k.lay.gains);

    // ------------------------------------------------------------ q/k/v product
    {
      ld_q(k, l, x, j, w, lane, aQ);
      if (!wg_wait(k, tid, KR2, x, kXcds, kPerXcd, pp_tag(k.tag0, l - 1, KR2), &stop, l - 1)) return;
      f4 acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (NT <= 2) {  // both steps' operands in flight before the norm's loads (wave 0)
        bf16x8 bh[2][NT][2], bl[2][NT][2];
#pragma unroll
        for (int s = 0; s < 2; ++s) load_b<NT>(xb, kH, 16 * w + 8 * s, lane, bh[s], bl[s]);
        rms_of<NPP>(ss, A.eps, rs, tid);
#pragma unroll
        for (int s = 0; s < 2; ++s) mfma_step<NT>(aQ[s], bh[s], bl[s], acc);
      } else {  // one step's operands in registers at a time
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          bf16x8 bh[NT][2], bl[NT][2];
          load_b<NT>(xb, kH, 16 * w + 8 * s, lane, bh, bl);
          if (s == 0) rms_of<NPP>(ss, A.eps, rs, tid);
          mfma_step<NT>(aQ[s], bh, bl, acc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) red[(w * NT + nt) * 64 + lane] = acc[nt];
      __syncthreads();
      const int t = tid;
      if (t < NT * 64) {
        const int nt = t >> 6, ln = t & 63;
        f4 o = red[(0 * NT + nt) * 64 + ln];
#pragma unroll
        for (int v = 1; v < 8; ++v) o += red[(v * NT + nt) * 64 + ln];
        const int n = 16 * nt + (ln & 15), r0 = 16 * j + 4 * (ln >> 4);
        const float sc = rs[n];
        const u4 val = {__float_as_uint(o[0] * sc), __float_as_uint(o[1] * sc), __float_as_uint(o[2] * sc),
                        __float_as_uint(o[3] * sc)};
        qr.st16((uint32_t)((n * kQRows + r0) * 4), val, plain);
      }
      wg_publish(k, KQ, pp_tag(k.tag0, l, KQ), plain, l);
    }

    // ------------------------------------------------------------ attention
    {
      if (!wg_wait(k, tid, KQ, x, kXcds, kPerXcd, pp_tag(k.tag0, l, KQ), &stop, l)) return;
      const int na = j, nb2 = j + kPerXcd;
      const bool va = na < m, vb = NPP > kPerXcd && nb2 < m;
      // padding positions of the O operand read zeros
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int n = u == 0 ? na : nb2;
        if (n >= m && n < NPP && tid < 64) {
          const int ch = tid & 31, part = tid >> 5;
          at.st16((uint32_t)(((ch * NPP + n) * 16) + part * kQpg * kD * NPP * 2), u4{0u, 0u, 0u, 0u}, plain);
        }
      }
      const int nmax = vb ? nb2 : (va ? na : -1);
      if (nmax >= 0) {
        // Wave w prepares the chunk's key and value rows w, w + 8, ... up to nmax (every
        // load issued before the first row's arithmetic), and waves 0..3 also query head
        // h = w & 1 of slot w >> 1: RMSNorm, rotary from the launch's table, bf16 rounding
        // of keys and values as the cache holds them.
        constexpr int RPW = NPP / 8;          // rows per wave at most
        constexpr int RB = RPW < 4 ? RPW : 4;  // rows per batch of loads
        const float* kn = G + kH + kD;
        const int qs_slot = w >> 1, qh = w & 1, qn_pos = qs_slot ? nb2 : na;
        const bool has_q = w < 4 && (qs_slot ? vb : va);
        float q0 = 0.f, q1 = 0.f;
        if (has_q) {
          q0 = __uint_as_float(qr.ld4((uint32_t)((qn_pos * kQRows + qh * kD + lane) * 4)));
          q1 = __uint_as_float(qr.ld4((uint32_t)((qn_pos * kQRows + qh * kD + lane + 64) * 4)));
        }
#pragma unroll
        for (int b0 = 0; b0 < RPW; b0 += RB) {
        float kv[RB][4];
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const int n = w + 8 * (b0 + u);
          const uint32_t o = (uint32_t)((n * kQRows + 2 * kD + lane) * 4);
          if (n <= nmax) {
            kv[u][0] = __uint_as_float(qr.ld4(o));
            kv[u][1] = __uint_as_float(qr.ld4(o + 64 * 4));
            kv[u][2] = __uint_as_float(qr.ld4(o + kD * 4));
            kv[u][3] = __uint_as_float(qr.ld4(o + (kD + 64) * 4));
          }
        }
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const int n = w + 8 * (b0 + u);
          if (n <= nmax) {
            float k0 = kv[u][0], k1 = kv[u][1];
            norm_rotate(kn, A.eps, rc[n][lane], rsn[n][lane], lane, k0, k1);
            const uint16_t kb0 = to_bf(k0), kb1 = to_bf(k1), vb0 = to_bf(kv[u][2]), vb1 = to_bf(kv[u][3]);
            S.kl[n][lane] = kb0;
            S.kl[n][lane + 64] = kb1;
            S.vl[n][lane] = vb0;
            S.vl[n][lane + 64] = vb1;
            if (n == na || n == nb2) {
              const size_t crow = (((size_t)l * kXcds + x) * A.max_seq + A.pos0 + n) * kD;
              A.kcache[crow + lane] = kb0;
              A.kcache[crow + lane + 64] = kb1;
              A.vcache[crow + lane] = vb0;
              A.vcache[crow + lane + 64] = vb1;
            }
          }
        }
        }
        if (has_q) {
          norm_rotate(G + kH, A.eps, rc[qn_pos][lane], rsn[qn_pos][lane], lane, q0, q1);
          const float qscale = rsqrtf((float)kD);
          S.qs[qs_slot][qh][lane] = q0 * qscale;
          S.qs[qs_slot][qh][lane + 64] = q1 * qscale;
        }
        __syncthreads();
        if (va) attend<NPP>(k, S, l, x, na, 0, at, plain, tid);
        if (vb) attend<NPP>(k, S, l, x, nb2, 1, at, plain, tid);
      }
      wg_publish(k, KA, pp_tag(k.tag0, l, KA), plain, l);
    }

    // ------------------------------------------------------------ O product (partial of KV block x)
    {
      constexpr int kSteps = kQpg * kD / 64;  // 4: waves 0..3, one operand step each
      const bool act = w < kSteps;
      if (act) ld_o(k, l, x, j, w, lane, aO);
      if (!wg_wait(k, tid, KA, x, kXcds, kPerXcd, pp_tag(k.tag0, l, KA), &stop, l)) return;
      if (act) {
        f4 acc[2][NT];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f4{0.f, 0.f, 0.f, 0.f};
        bf16x8 bh[NT][2], bl[NT][2];
        load_b<NT>(at, kQpg * kD, 8 * w, lane, bh, bl);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) mfma_step<NT>(aO[rt], bh, bl, acc[rt]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) red[((w * 2 + rt) * NT + nt) * 64 + lane] = acc[rt][nt];
      }
      __syncthreads();
      const int t = tid;
      if (t < 2 * NT * 64) {
        const int rr = t / (NT * 64), nt = (t >> 6) % NT, ln = t & 63;
        f4 o = red[((0 * 2 + rr) * NT + nt) * 64 + ln];
#pragma unroll
        for (int v = 1; v < kSteps; ++v) o += red[((v * 2 + rr) * NT + nt) * 64 + ln];
        const int n = 16 * nt + (ln & 15), r0 = 16 * rr + 4 * (ln >> 4);
        const u4 val = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
        op.st16((uint32_t)((((x * kPerXcd + j) * NPP + n) * kCw + r0) * 4), val, false);
      }
      wg_publish(k, KO, pp_tag(k.tag0, l, KO), false, l);
    }

    // ------------------------------------------------------------ residual after attention
    {
      if (!wg_wait(k, tid, KO, kXcds * j, 1, kXcds, pp_tag(k.tag0, l, KO), &stop, l)) return;
      float g8[8];
      load_gains(G, j, tid, g8);  // in flight with the partials' loads
      add_partials<NPP>(xres, op, j, tid);
      __syncthreads();
      publish_residual<NPP>(xres, g8, j, xp, ss2, plain, tid);
      wg_publish(k, KR1, pp_tag(k.tag0, l, KR1), plain, l);
    }

    // ------------------------------------------------------------ gate/up product and SwiGLU
    {
      ld_g(k, l, x, j, w, lane, aG);
      if (!wg_wait(k, tid, KR1, x, kXcds, kPerXcd, pp_tag(k.tag0, l, KR1), &stop, l)) return;
      f4 acc[2][NT];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (NT <= 2) {  // both steps' operands in flight before the norm's loads
        bf16x8 bh[2][NT][2], bl[2][NT][2];
#pragma unroll
        for (int s = 0; s < 2; ++s) load_b<NT>(xp, kH, 16 * w + 8 * s, lane, bh[s], bl[s]);
        rms_of<NPP>(ss2, A.eps, rs, tid);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) mfma_step<NT>(aG[rt][s], bh[s], bl[s], acc[rt]);
      } else {  // one step's operands in registers at a time
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          bf16x8 bh[NT][2], bl[NT][2];
          load_b<NT>(xp, kH, 16 * w + 8 * s, lane, bh, bl);
          if (s == 0) rms_of<NPP>(ss2, A.eps, rs, tid);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) mfma_step<NT>(aG[rt][s], bh, bl, acc[rt]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) red[((w * 2 + rt) * NT + nt) * 64 + lane] = acc[rt][nt];
      __syncthreads();
      const int t = tid;
      if (t < 2 * NT * 64) {
        const int rt = t / (NT * 64), nt = (t >> 6) % NT, ln = t & 63;
        f4 o = red[((0 * 2 + rt) * NT + nt) * 64 + ln];
#pragma unroll
        for (int v = 1; v < 8; ++v) o += red[((v * 2 + rt) * NT + nt) * 64 + ln];
        const int n = 16 * nt + (ln & 15), r0 = 16 * rt + 4 * (ln >> 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (r0 + e < 2 * kHalf) gu[n][r0 + e] = o[e];
      }
      __syncthreads();
#pragma nounroll
      for (int u = t; u < NPP * kHalf; u += kPpThreads) {
        const int n = u / kHalf, c = u % kHalf;
        const float r = rs[n];
        const float gr = gu[n][c] * r;
        const float hv = gr / (1.f + __expf(-gr)) * (gu[n][kHalf + c] * r);
        const uint16_t hh = to_bf(hv), hl = to_bf(hv - from_bf(hh));
        const int col = kHalf * j + c;
        const uint32_t off = (uint32_t)((((col >> 3) * NPP + n) * 8 + (col & 7)) * 2);
        hs.st2(off, hh, plain);
        hs.st2(off + (uint32_t)(kIx * NPP * 2), hl, plain);
      }
      wg_publish(k, KG, pp_tag(k.tag0, l, KG), plain, l);
    }

    // ------------------------------------------------------------ down product (partial of slice x)
    {
      constexpr int kSteps = kIx / 64;  // 6: waves 0..5, one operand step each
      const bool act = w < kSteps;
      if (NT < 4 && act) ld_d(k, l, x, j, w, lane, aD);
      if (!wg_wait(k, tid, KG, x, kXcds, kPerXcd, pp_tag(k.tag0, l, KG), &stop, l)) return;
      if (NT >= 4 && act) ld_d(k, l, x, j, w, lane, aD);
      if (act) {
        f4 acc[2][NT];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f4{0.f, 0.f, 0.f, 0.f};
        bf16x8 bh[NT][2], bl[NT][2];
        load_b<NT>(hs, kIx, 8 * w, lane, bh, bl);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) mfma_step<NT>(aD[rt], bh, bl, acc[rt]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) red[((w * 2 + rt) * NT + nt) * 64 + lane] = acc[rt][nt];
      }
      __syncthreads();
      const int t = tid;
      if (t < 2 * NT * 64) {
        const int rr = t / (NT * 64), nt = (t >> 6) % NT, ln = t & 63;
        f4 o = red[((0 * 2 + rr) * NT + nt) * 64 + ln];
#pragma unroll
        for (int v = 1; v < kSteps; ++v) o += red[((v * 2 + rr) * NT + nt) * 64 + ln];
        const int n = 16 * nt + (ln & 15), r0 = 16 * rr + 4 * (ln >> 4);
        const u4 val = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
        dp.st16((uint32_t)((((x * kPerXcd + j) * NPP + n) * kCw + r0) * 4), val, false);
      }
      wg_publish(k, KD, pp_tag(k.tag0, l, KD), false, l);
    }

    // ------------------------------------------------------------ residual after the MLP
    {
      if (!wg_wait(k, tid, KD, kXcds * j, 1, kXcds, pp_tag(k.tag0, l, KD), &stop, l)) return;
      float g8[8];
      load_gains(G + kH + 2 * kD, j, tid, g8);  // in flight with the partials' loads
      add_partials<NPP>(xres, dp, j, tid);
      __syncthreads();
      const int t = tid;
      if (x == 0 && t < NPP * (kCw / 4)) {  // one XCD's replica: the layer output, and after the last layer the residual the LM head reads
        const int n = t / (kCw / 4), c4 = t % (kCw / 4), col = kCw * j + 4 * c4;
        if (n < m) {
          if (A.dbg_hidden)
#pragma unroll
            for (int e = 0; e < 4; ++e) A.dbg_hidden[((size_t)n * (L + 1) + l + 1) * kH + col + e] = xres[n][4 * c4 + e];
          if (l + 1 == L)
            *reinterpret_cast<float4*>(A.x + (size_t)n * kH + col) =
                make_float4(xres[n][4 * c4], xres[n][4 * c4 + 1], xres[n][4 * c4 + 2], xres[n][4 * c4 + 3]);
        }
      }
      if (l + 1 < L) {
        publish_residual<NPP>(xres, g8, j, xb, ss, plain, tid);
        wg_publish(k, KR2, pp_tag(k.tag0, l, KR2), plain, l);
      }
    }
  }
}

__global__ void pp_clear_kernel(unsigned long long* flags, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) flags[i] = 0ull;
}

template <int NT>
int launch_nt(PpK& k, hipStream_t st) {
  static int occ = -1;
  if (occ < 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void*)pp_kernel<NT>, kPpThreads, 0) != hipSuccess) return -1;
    occ = nb;
  }
  if (occ < 1) return -1;
  void* args[] = {&k};
  return hipLaunchCooperativeKernel((const void*)pp_kernel<NT>, dim3(kGrid), dim3(kPpThreads), args, 0, st) == hipSuccess
             ? 0
             : -1;
}

}  // namespace

bool pp_supported(int H, int NQ, int NKV, int D, int I) {
  return H == kH && I == kI && D == kD && NKV == kXcds && NQ == kQpg * NKV;
}

size_t pp_layout(int H, int NQ, int NKV, int D, int I, size_t offs[10]) {
  if (!pp_supported(H, NQ, NKV, D, I)) return 0;
  const size_t P = kPrefillChunk;
  const size_t sizes[10] = {
      (size_t)kPpKinds * kGrid * 8,          // flags
      (size_t)kXcds * 2 * kH * P * 2,        // xb
      (size_t)kXcds * 2 * kH * P * 2,        // xp
      (size_t)kXcds * kPerXcd * P * 4,       // ss
      (size_t)kXcds * kPerXcd * P * 4,       // ss2
      (size_t)kXcds * P * kQRows * 4,        // qr
      (size_t)kXcds * 2 * kQpg * kD * P * 2, // at
      (size_t)kXcds * kPerXcd * P * kCw * 4, // op
      (size_t)kXcds * 2 * kIx * P * 2,       // hs
      (size_t)kXcds * kPerXcd * P * kCw * 4, // dp
  };
  size_t off = 0;
  for (int r = 0; r < 10; ++r) {
    offs[r] = off;
    off += (sizes[r] + 255) / 256 * 256;
  }
  return off;
}

int launch_pp_clear(unsigned long long* flags, void* stream) {
  hipLaunchKernelGGL(pp_clear_kernel, dim3(8), dim3(256), 0, (hipStream_t)stream, flags, kPpKinds * kGrid);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_prefill_persistent(const PfArgs& A, const PpBufs& B, const uint8_t* layers, const LayerLayout& lay,
                              uint32_t tag0, uint32_t spin_limit, uint32_t* abort_flag, unsigned long long* dbg_phase,
                              void* stream) {
  if (!pp_supported(A.H, A.NQ, A.NKV, A.D, A.I) || A.m <= 0 || A.m > A.npp || A.npp % 16 || A.npp > kPrefillChunk ||
      A.pos0 + A.m > kPpMaxKeys)
    return -1;
  PpK k{A, B, layers, lay, tag0, spin_limit, abort_flag, dbg_phase};
  hipStream_t st = (hipStream_t)stream;
  switch (A.npp / 16) {
    case 1: return launch_nt<1>(k, st);
    case 2: return launch_nt<2>(k, st);
    case 3: return launch_nt<3>(k, st);
    case 4: return launch_nt<4>(k, st);
  }
  return -1;
}

}  // namespace mk
