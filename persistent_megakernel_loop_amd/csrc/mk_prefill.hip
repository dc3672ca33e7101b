// Batched prompt prefill.
//
// The persistent decode kernel runs one position per pass over the weights, so a
// prompt of P positions costs P passes.  Every prompt position is known up front,
// which makes the prompt a batch: each layer's projections become
// matrix products with P columns, and the weights stream once per chunk of up to 64
// positions instead of once per position.  The causal mask keeps the result the same
// as the position-by-position run (up to rounding order): position p attends to
// cache entries 0..p, all of which are written before the chunk's attention runs.
//
// One chunk, per layer, as a short sequence of ordinary kernels on the handle's
// stream:
//   input rows and RMSNorm (layer 0) or residual + RMSNorm (later layers)
//   QKV product -> per-head q/k RMSNorm, rotary embedding, cache write
//   causal attention: one workgroup per (position, KV group) for short contexts, key
//   ranges on the matrix cores and their merge behind a long cache
//   O product -> residual + post-attention RMSNorm
//   gate/up product -> SwiGLU
//   down product -> residual + next input RMSNorm
// The products read the weight tiles of the persistent kernel's arena as they are
// (no second copy of the weights) and run on the matrix cores: 16x16x32 bf16 MFMA
// with the activations split into a bf16 high and low part (two products per tile),
// so the activations keep about 16 significant bits, as the fp32 dot products of the
// decode path do up to rounding.  After the last chunk, the LM head over the last
// position and a greedy argmax produce the first id and publish it as the persistent
// kernel would (device output, feedback id, pinned mirror, progress word).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"
#include "mk_prefill.h"

namespace mk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Split-activation layout of a K-column input for npp positions: element k of
// position n at [(k/8)*npp + n][k%8] (the high parts), the low parts K*npp elements
// further.  Eight consecutive columns of one position are one 16-byte chunk, and
// the 16 positions of a tile are 16 consecutive chunks.
__device__ __forceinline__ void store_split8(uint16_t* xs, int K, int npp, int n, int c, const float v[8]) {
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t h0 = to_bf16(v[2 * e]), h1 = to_bf16(v[2 * e + 1]);
    const uint16_t l0 = to_bf16(v[2 * e] - from_bf16(h0)), l1 = to_bf16(v[2 * e + 1] - from_bf16(h1));
    hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    lo[e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
  const size_t off = ((size_t)c * npp + n) * 8;
  *reinterpret_cast<uint4*>(xs + off) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  *reinterpret_cast<uint4*>(xs + (size_t)K * npp + off) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

__device__ __forceinline__ void zero_split8(uint16_t* xs, int K, int npp, int n, int c) {
  const size_t off = ((size_t)c * npp + n) * 8;
  *reinterpret_cast<uint4*>(xs + off) = make_uint4(0, 0, 0, 0);
  *reinterpret_cast<uint4*>(xs + (size_t)K * npp + off) = make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// The RMSNorm feeding a product is taken apart as the decode path does: the product's
// input is gains * x (split), and its consumer scales the result by the row's 1/rms,
// read from per-512-column sums of squares.  A residual row is then written by H/512
// one-wave blocks with no reduction across the row.
__device__ __forceinline__ float row_rs(const PfArgs& A, int n) {
  const int nb = A.H / 512;
  float ss = 0.f;
  for (int b = 0; b < nb; ++b) ss += A.ss[n * nb + b];
  return rsqrtf(ss / (float)A.H + A.eps);
}

// Columns 8c .. 8c+7 of row n (values v): gains * x split for the next product, and
// the squares summed over the block into ss[n][blockIdx.y].
__device__ __forceinline__ void gain_split(const PfArgs& A, const float* g, int n, int c, const float v[8]) {
  float gv[8], sq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    gv[e] = g[8 * c + e] * v[e];
    sq = fmaf(v[e], v[e], sq);
  }
  store_split8(A.xs, A.H, A.npp, n, c, gv);
  sq = wsum(sq);
  if (threadIdx.x == 0) A.ss[n * (A.H / 512) + blockIdx.y] = sq;
}

// ------------------------------------------------------------------ input rows
// grid (npp, H/512), 64 threads; thread t of block (n, b) takes columns 8(64b + t) .. +7.
__global__ __launch_bounds__(64) void pf_input_kernel(PfArgs A) {
  const int n = blockIdx.x, H = A.H, c = blockIdx.y * 64 + threadIdx.x;
  if (n >= A.m) { zero_split8(A.xs, H, A.npp, n, c); return; }
  const int p = A.pos0 + n;
  int id = A.ids[n];
  if (id >= A.vocab || (id < 0 && A.rows == nullptr)) {  // flagged and read as id 0
    if (threadIdx.x == 0 && blockIdx.y == 0)
      __hip_atomic_fetch_or(A.err, DEV_ERR_ID, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    id = 0;
  }
  if (blockIdx.y == 0 && (int)threadIdx.x < A.n_sections) {
    const int v = A.pos3 ? A.pos3[n * 3 + threadIdx.x] : p;
    if (v < 0 || v >= A.rope_positions)
      __hip_atomic_fetch_or(A.err, DEV_ERR_POS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  float v[8];
  if (id >= 0) {
    const uint4 u = *reinterpret_cast<const uint4*>(A.embed + (size_t)id * H + 8 * c);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    load8(A.rows + (size_t)n * H + 8 * c, v);
  }
  store8(A.x + (size_t)n * H + 8 * c, v);
  if (A.dbg_hidden) store8(A.dbg_hidden + (size_t)n * (A.L + 1) * H + 8 * c, v);
  gain_split(A, A.in_norm0, n, c, v);
}

// ------------------------------------------------------------------ products
// part[ks][n][r] = sum over the ks-th run of WK*KC columns of W[r][k] * X[n][k].
// Weight element (r, k) sits at w[(k/KB)*R*KB + r*KB + k%KB] (KB = K for a plain
// row-major matrix; the O and down tiles are K-blocked per KV group and per MLP
// slice).  A workgroup of WK waves takes 32 rows x 16*NT positions over WK*KC
// columns, wave w the w-th run of KC = 64*S columns; the waves' results are summed
// in LDS in wave order and written once.  Per 64 columns, lane group q (lanes
// 16q..16q+15) holds columns 16q..16q+15 of 16 rows as two 8-column halves, and the
// activations of 16 positions over the same columns, so that each 16x16x32 MFMA pairs
// operands over the same 32 columns whatever order the hardware gives them inside
// the instruction.  The result tile has 4 consecutive rows per lane (rows 4q..4q+3 of
// the tile, position lane%16).
template <int NT, int S>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void pf_gemm_kernel(
    const uint16_t* __restrict__ w, int R, int KB, int K, const uint16_t* __restrict__ xs, float* __restrict__ part) {
  constexpr int NPP = 16 * NT, KC = 64 * S;
  __shared__ f4 red[3][2][NT][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, WK = blockDim.x >> 6;
  const int groups = R / 32;
  const int rg = blockIdx.x % groups, ks = blockIdx.x / groups;
  const int k0 = (ks * WK + wv) * KC, blk = k0 / KB, kk0 = k0 % KB;
  const int q = lane >> 4, i16 = lane & 15;
  const uint16_t* w0 = w + (size_t)blk * R * KB + (size_t)(rg * 32 + i16) * KB + kk0 + 16 * q;
  const uint16_t* w1 = w0 + (size_t)16 * KB;
  const uint16_t* xh = xs + ((size_t)(k0 / 8 + 2 * q) * NPP + i16) * 8;
  const uint16_t* xl = xh + (size_t)K * NPP;
  bf16x8 a[S][2][2];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      a[s][0][hf] = *reinterpret_cast<const bf16x8*>(w0 + s * 64 + hf * 8);
      a[s][1][hf] = *reinterpret_cast<const bf16x8*>(w1 + s * 64 + hf * 8);
    }
  f4 acc[2][NT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f4{0.f, 0.f, 0.f, 0.f};
  // The activations of SG column steps are loaded together (16 NT SG VGPRs, at most 128),
  // the first group's behind the weights: every load of a group is in flight before the
  // first product waits on one.
  constexpr int SG = NT * S <= 8 ? S : (8 / NT > 0 ? 8 / NT : 1);
  static_assert(S % SG == 0, "whole groups of column steps");
#pragma unroll
  for (int s0 = 0; s0 < S; s0 += SG) {
    bf16x8 bh[SG][NT][2], bl[SG][NT][2];
#pragma unroll
    for (int sg = 0; sg < SG; ++sg)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const size_t off = ((size_t)((s0 + sg) * 8 + hf) * NPP + nt * 16) * 8;
          bh[sg][nt][hf] = *reinterpret_cast<const bf16x8*>(xh + off);
          bl[sg][nt][hf] = *reinterpret_cast<const bf16x8*>(xl + off);
        }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sg = 0; sg < SG; ++sg)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int s = s0 + sg;
            acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s][rt][hf], bh[sg][nt][hf], acc[rt][nt], 0, 0, 0);
            acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s][rt][hf], bl[sg][nt][hf], acc[rt][nt], 0, 0, 0);
          }
  }
  if (wv > 0) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) red[wv - 1][rt][nt][lane] = acc[rt][nt];
  }
  __syncthreads();
  if (wv > 0) return;
  for (int v = 1; v < WK; ++v)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rt][nt] += red[v - 1][rt][nt][lane];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<f4*>(part + ((size_t)ks * NPP + nt * 16 + i16) * R + rg * 32 + rt * 16 + 4 * q) = acc[rt][nt];
}

// ------------------------------------------------------------------ q, k, v
// One workgroup per (KV group g, position n); wave h < QPG takes q head h, wave QPG
// the key, wave QPG+1 the value.  Lane i holds elements i and i + 64 of its head,
// which are rotary pair i (head dim 128).
__global__ __launch_bounds__(256) void pf_qkv_kernel(PfArgs A, int l, const float* G, int ks) {
  constexpr int D = 128, QPG = 2;
  const int g = blockIdx.x, n = blockIdx.y, h = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int p = A.pos0 + n;
  const int R = A.NKV * (QPG + 2) * D;
  const int row = g * (QPG + 2) * D + h * D + lane;
  // the rotary pair's cos/sin first: their loads depend on the position stream's, and
  // this way both are in flight with the partials'
  const int sct = lane < A.sec_end0 ? 0 : (lane < A.sec_end1 ? 1 : 2);
  int ps = A.pos3 ? A.pos3[n * 3 + sct] : p;
  ps = (ps < 0 || ps >= A.rope_positions) ? 0 : ps;
  const float c = A.rope_cos[(size_t)ps * (D / 2) + lane], sn = A.rope_sin[(size_t)ps * (D / 2) + lane];
  float a0 = 0.f, a1 = 0.f;
  for (int s = 0; s < ks; ++s) {
    const float* pp = A.part + ((size_t)s * A.npp + n) * R + row;
    a0 += pp[0];
    a1 += pp[64];
  }
  const float xr = row_rs(A, n);  // the input norm's 1/rms
  a0 *= xr;
  a1 *= xr;
  const size_t crow = (((size_t)l * A.NKV + g) * A.max_seq + p) * D;
  if (h <= QPG) {
    const float* gn = G + A.H + (h < QPG ? 0 : D);
    const float ss = wsum(fmaf(a1, a1, a0 * a0));
    const float rs = rsqrtf(ss / (float)D + A.eps);
    const float n0 = gn[lane] * (a0 * rs), n1 = gn[lane + 64] * (a1 * rs);
    const float o0 = n0 * c - n1 * sn, o1 = n1 * c + n0 * sn;
    if (h < QPG) {
      const float qscale = rsqrtf((float)D);
      float* qo = A.q + ((size_t)n * A.NQ + g * QPG + h) * D;
      qo[lane] = o0 * qscale;
      qo[lane + 64] = o1 * qscale;
    } else {
      A.kcache[crow + lane] = to_bf16(o0);
      A.kcache[crow + lane + 64] = to_bf16(o1);
    }
  } else {
    A.vcache[crow + lane] = to_bf16(a0);
    A.vcache[crow + lane + 64] = to_bf16(a1);
  }
}

// ------------------------------------------------------------------ attention
// One workgroup of kPfAttnWaves waves per (KV group g, position n) over cache positions
// 0..p: wave w takes the 64-key blocks w, w + kPfAttnWaves, ...; lane j of a block
// scores key j against the group's QPG query heads, the block's softmax weights go
// through LDS, and the values are read as whole rows (lane i holds dims 2i, 2i+1).
// The waves' running maxima, sums and outputs merge in LDS; the result goes out split
// for the O product.  Behind a long cache each wave's blocks form a chain of dependent
// loads, so more waves per workgroup shorten it.

// Eight bf16 cache elements widened to float32.
__device__ __forceinline__ void cvt_row8(const uint4 r, float v[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}

constexpr int kPfAttnWaves = 8;  // two per SIMD: each wave may use 256 VGPRs

__global__ __launch_bounds__(64 * kPfAttnWaves) void pf_attn_kernel(PfArgs A, int l) {
  constexpr int D = 128, QPG = 2, NW = kPfAttnWaves;
  __shared__ float qs[QPG][D];
  __shared__ float pw[NW][QPG][64];
  __shared__ float mw[NW][QPG], lw[NW][QPG];
  __shared__ float aw[NW][QPG][D];
  const int g = blockIdx.x, n = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int K = A.NQ * D;
  if (n >= A.m) {  // padding columns of the O product
    if (w < QPG) {
      const int e = (g * QPG + w) * D + 2 * lane;
      const size_t off = ((size_t)(e / 8) * A.npp + n) * 8 + e % 8;
      *reinterpret_cast<uint32_t*>(A.xs + off) = 0u;
      *reinterpret_cast<uint32_t*>(A.xs + (size_t)K * A.npp + off) = 0u;
    }
    return;
  }
  const int p = A.pos0 + n, nkeys = p + 1;
  const size_t cbase = ((size_t)l * A.NKV + g) * A.max_seq * D;
  // A block's key row (the whole row in flight at once, converted after) and its first 32
  // value rows (2 dims per lane; rows past the block's last key read that key's row, with
  // weight 0) are issued together; for the wave's first block, before q is read, so the
  // three loads overlap.
  uint4 kr[D / 8];
  uint32_t vr[32];
  auto load_block = [&](int kb) {
    const int j = kb * 64 + lane;
    const size_t krow = cbase + (size_t)(j < nkeys ? j : p) * D;
#pragma unroll
    for (int j8 = 0; j8 < D / 8; ++j8) kr[j8] = *reinterpret_cast<const uint4*>(A.kcache + krow + 8 * j8);
    const int nb = min(64, nkeys - kb * 64);
#pragma unroll
    for (int e = 0; e < 32; ++e)
      vr[e] = *reinterpret_cast<const uint32_t*>(A.vcache + cbase + (size_t)(kb * 64 + min(e, nb - 1)) * D + 2 * lane);
  };
  if (w * 64 < nkeys) load_block(w);
  for (int i = threadIdx.x; i < QPG * D; i += blockDim.x)
    qs[i / D][i % D] = A.q[((size_t)n * A.NQ + g * QPG) * D + i];
  __syncthreads();
  float M[QPG], Ls[QPG], acc[QPG][2];
#pragma unroll
  for (int h = 0; h < QPG; ++h) { M[h] = -INFINITY; Ls[h] = 0.f; acc[h][0] = acc[h][1] = 0.f; }
  for (int kb = w; kb * 64 < nkeys; kb += NW) {
    if (kb != w) load_block(kb);
    const int j = kb * 64 + lane;
    const bool valid = j < nkeys;
    float s[QPG];
#pragma unroll
    for (int h = 0; h < QPG; ++h) s[h] = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j8 = 0; j8 < D / 8; ++j8) {
      float kv[8];
      cvt_row8(kr[j8], kv);
#pragma unroll
      for (int h = 0; h < QPG; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) s[h] = fmaf(qs[h][8 * j8 + e], kv[e], s[h]);
    }
#pragma unroll
    for (int h = 0; h < QPG; ++h) {
      const float sv = valid ? s[h] : -INFINITY;
      const float mn = fmaxf(M[h], wmax(sv));  // finite: key kb*64 is valid
      const float corr = __expf(M[h] - mn);    // 0 while M is still -inf
      const float pr = valid ? __expf(sv - mn) : 0.f;
      Ls[h] = Ls[h] * corr + wsum(pr);
      acc[h][0] *= corr;
      acc[h][1] *= corr;
      M[h] = mn;
      pw[w][h][lane] = pr;
    }
    // the block's weights are read back by every lane of this wave (LDS accesses of
    // one wave complete in order)
    __builtin_amdgcn_wave_barrier();
    const int nb = min(64, nkeys - kb * 64);
    // value rows 0..31 of the block (loaded with its key row), then 32..63 if it has them
#pragma unroll
    for (int e = 0; e < 32; ++e)
#pragma unroll
      for (int h = 0; h < QPG; ++h) {
        const float pu = e < nb ? pw[w][h][e] : 0.f;
        acc[h][0] = fmaf(pu, __uint_as_float(vr[e] << 16), acc[h][0]);
        acc[h][1] = fmaf(pu, __uint_as_float(vr[e] & 0xffff0000u), acc[h][1]);
      }
    if (nb > 32) {  // 32 value rows in flight at once
      float v0[32], v1[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int u = min(32 + e, nb - 1);  // past the block's last key: weight 0, row in range
        const uint32_t vv = *reinterpret_cast<const uint32_t*>(A.vcache + cbase + (size_t)(kb * 64 + u) * D + 2 * lane);
        v0[e] = __uint_as_float(vv << 16);
        v1[e] = __uint_as_float(vv & 0xffff0000u);
      }
#pragma unroll
      for (int e = 0; e < 32; ++e)
#pragma unroll
        for (int h = 0; h < QPG; ++h) {
          const float pu = 32 + e < nb ? pw[w][h][32 + e] : 0.f;
          acc[h][0] = fmaf(pu, v0[e], acc[h][0]);
          acc[h][1] = fmaf(pu, v1[e], acc[h][1]);
        }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int h = 0; h < QPG; ++h) {
    if (lane == 0) { mw[w][h] = M[h]; lw[w][h] = Ls[h]; }
    aw[w][h][2 * lane] = acc[h][0];
    aw[w][h][2 * lane + 1] = acc[h][1];
  }
  __syncthreads();
  if (w < QPG) {
    const int h = w;
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) mx = fmaxf(mx, mw[v][h]);
    float f[NW], lsum = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      f[v] = mw[v][h] == -INFINITY ? 0.f : __expf(mw[v][h] - mx);
      lsum = fmaf(f[v], lw[v][h], lsum);
    }
    const float inv = 1.f / lsum;
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      o0 = fmaf(f[v], aw[v][h][2 * lane], o0);
      o1 = fmaf(f[v], aw[v][h][2 * lane + 1], o1);
    }
    o0 *= inv;
    o1 *= inv;
    const uint16_t h0 = to_bf16(o0), h1 = to_bf16(o1);
    const uint16_t l0 = to_bf16(o0 - from_bf16(h0)), l1 = to_bf16(o1 - from_bf16(h1));
    const int e = (g * QPG + h) * D + 2 * lane;
    const size_t off = ((size_t)(e / 8) * A.npp + n) * 8 + e % 8;
    *reinterpret_cast<uint32_t*>(A.xs + off) = (uint32_t)h0 | ((uint32_t)h1 << 16);
    *reinterpret_cast<uint32_t*>(A.xs + (size_t)K * A.npp + off) = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
}

// ------------------------------------------------------------------ attention (flash)
// One workgroup of 4 waves per (KV group g, key range s) takes every query row of the
// chunk (row 2n + h: position n, head h of the group) against keys [s*SK, s*SK + SK)
// clipped to the chunk's last position, 32 keys at a time:
//   S = Q K^T on the matrix cores (16 rows x 16 keys per MFMA tile, the queries split
//   into bf16 high and low parts, the keys exact in bf16); causal mask (row n sees keys
//   up to pos0 + n); a running maximum and sum per row across the range (a row's 16
//   keys of a tile sit in 16 lanes, reduced with xor shuffles);
//   P = exp(S - max) through LDS as bf16 high/low parts, and the value tile transposed
//   into LDS, so that O += P V is on the matrix cores too.
// Wave w takes row tiles w, w + 4, ... (16 rows each).  Each range leaves, per row, its
// maximum, sum and unnormalised output; pf_attn_combine_kernel merges the ranges in
// order.  Rows with no visible key in a range leave maximum -inf and sum 0.
constexpr int kFlashKeys = 128;  // keys per range, widened so that there are at most kFlashRanges
// Contexts up to this many keys take pf_attn_kernel instead (256 workgroups and no merge
// launch; measured faster up to about 1000-2000 keys, the key ranges faster beyond).
constexpr int kFlashMinKeys = 2048;

__device__ __forceinline__ bf16x8 bf16x8_of(const uint4 u) { return __builtin_bit_cast(bf16x8, u); }

template <int NT>
__global__ __launch_bounds__(256) void pf_flash_kernel(PfArgs A, int l, int sk) {
  constexpr int D = 128, QPG = 2, NPP = 16 * NT, ROWS = QPG * NPP, RT = ROWS / 16;
  __shared__ __align__(16) uint16_t vt[D][32 + 8];  // value tile transposed: [dim][key] (+8: bank spread)
  __shared__ __align__(16) uint16_t ph[4][16][32 + 8], pl[4][16][32 + 8];  // per wave: P high/low parts
  const int g = blockIdx.x, s = blockIdx.y, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q4 = lane >> 4, i16 = lane & 15;
  const int kend = A.pos0 + A.m;                 // keys [0, kend) exist
  const int k0 = s * sk, k1 = min(kend, k0 + sk);
  const size_t cbase = ((size_t)l * A.NKV + g) * A.max_seq * D;
  float* out = A.att + ((size_t)(g * kFlashRanges + s) * ROWS) * (D + 2);
  // this wave's row tiles (at most 2 for 64 positions)
  constexpr int MT = (RT + 3) / 4;
  bf16x8 qh[MT][4], ql[MT][4];
  f4 o[MT][8];
  float m[MT][4], ls[MT][4];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int rt = wv + 4 * t;
    const int row = rt * 16 + i16, n = row >> 1, h = row & 1;
    const bool live = rt < RT && n < A.m;
    const float* qrow = A.q + ((size_t)n * A.NQ + g * QPG + h) * D;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float v[8];
      if (live) load8(qrow + kk * 32 + 8 * q4, v);
      else for (int e = 0; e < 8; ++e) v[e] = 0.f;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t h0 = to_bf16(v[2 * e]), h1 = to_bf16(v[2 * e + 1]);
        hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[e] = (uint32_t)to_bf16(v[2 * e] - from_bf16(h0)) | ((uint32_t)to_bf16(v[2 * e + 1] - from_bf16(h1)) << 16);
      }
      qh[t][kk] = bf16x8_of(make_uint4(hi[0], hi[1], hi[2], hi[3]));
      ql[t][kk] = bf16x8_of(make_uint4(lo[0], lo[1], lo[2], lo[3]));
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) o[t][d] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) { m[t][e] = -INFINITY; ls[t][e] = 0.f; }
  }
  for (int kt = k0; kt < k1; kt += 32) {
    // the value tile, transposed into LDS by the whole workgroup (rows past the range
    // re-read its last key: their weights are 0)
    __syncthreads();
    {
      const int key = threadIdx.x >> 4, d0 = 8 * (threadIdx.x & 15);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int kk = key + 16 * half;
        const uint4 u = *reinterpret_cast<const uint4*>(A.vcache + cbase + (size_t)min(kt + kk, k1 - 1) * D + d0);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vt[d0 + 2 * e][kk] = (uint16_t)(w[e] & 0xffffu);
          vt[d0 + 2 * e + 1][kk] = (uint16_t)(w[e] >> 16);
        }
      }
    }
    __syncthreads();
    // key fragments: lane (i16, q4) holds key kt + 16c + i16, dims 32kk + 8q4 .. + 7
    bf16x8 kf[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int key = min(kt + 16 * c + i16, k1 - 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kf[c][kk] = bf16x8_of(*reinterpret_cast<const uint4*>(A.kcache + cbase + (size_t)key * D + kk * 32 + 8 * q4));
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int rt = wv + 4 * t;
      if (rt >= RT) break;
      f4 sc[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        sc[c] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          sc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[t][kk], kf[c][kk], sc[c], 0, 0, 0);
          sc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[t][kk], kf[c][kk], sc[c], 0, 0, 0);
        }
      }
      // lane holds rows 4q4 + e of the tile, keys kt + 16c + i16
      float p[2][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = (rt * 16 + 4 * q4 + e) >> 1;
        const int kmax = A.pos0 + n;  // causal: keys up to the row's own position
        float sv[2], mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int key = kt + 16 * c + i16;
          sv[c] = (key < k1 && key <= kmax) ? sc[c][e] : -INFINITY;
          mx = fmaxf(mx, sv[c]);
        }
#pragma unroll
        for (int x = 1; x < 16; x <<= 1) mx = fmaxf(mx, __shfl_xor(mx, x, 64));
        const float mn = fmaxf(m[t][e], mx);
        const bool none = mn == -INFINITY;  // no visible key yet: nothing to add
        const float corr = none ? 1.f : __expf(m[t][e] - mn);
        float sum = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          p[c][e] = (none || sv[c] == -INFINITY) ? 0.f : __expf(sv[c] - mn);
          sum += p[c][e];
        }
#pragma unroll
        for (int x = 1; x < 16; x <<= 1) sum += __shfl_xor(sum, x, 64);
        ls[t][e] = ls[t][e] * corr + sum;
        m[t][e] = mn;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[t][d][e] *= corr;
      }
      // P into LDS (this wave's area), high and low parts, [row][key]
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint16_t hb = to_bf16(p[c][e]);
          ph[wv][4 * q4 + e][16 * c + i16] = hb;
          pl[wv][4 * q4 + e][16 * c + i16] = to_bf16(p[c][e] - from_bf16(hb));
        }
      __builtin_amdgcn_wave_barrier();
      // A fragments of P: lane (i16, q4) holds row i16, keys 8q4 .. 8q4 + 7
      const bf16x8 pa = bf16x8_of(*reinterpret_cast<const uint4*>(&ph[wv][i16][8 * q4]));
      const bf16x8 pb = bf16x8_of(*reinterpret_cast<const uint4*>(&pl[wv][i16][8 * q4]));
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        // B fragment of V: lane (i16, q4) holds dim 16d + i16, keys 8q4 .. 8q4 + 7
        const bf16x8 vb = bf16x8_of(*reinterpret_cast<const uint4*>(&vt[16 * d + i16][8 * q4]));
        o[t][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[t][d], 0, 0, 0);
        o[t][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb, vb, o[t][d], 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  // this range's partials: per row its maximum, sum and unnormalised output
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int rt = wv + 4 * t;
    if (rt >= RT) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float* r = out + (size_t)(rt * 16 + 4 * q4 + e) * (D + 2);
      if (i16 == 0) { r[0] = m[t][e]; r[1] = ls[t][e]; }
#pragma unroll
      for (int d = 0; d < 8; ++d) r[2 + 16 * d + i16] = o[t][d][e];
    }
  }
}

// Merge of the key ranges for (KV group g, position n): per head, the ranges' outputs
// weighted by exp(max_s - max) over the total sum, in range order; split for the O
// product (padding positions: zeros).
__global__ __launch_bounds__(256) void pf_attn_combine_kernel(PfArgs A, int n_ranges) {
  constexpr int D = 128, QPG = 2;
  const int g = blockIdx.x, n = blockIdx.y, h = threadIdx.x >> 7, d = threadIdx.x & 127;
  const int K = A.NQ * D, ROWS = QPG * A.npp;
  const int e = (g * QPG + h) * D + d;
  const size_t off = ((size_t)(e / 8) * A.npp + n) * 8 + e % 8;
  if (n >= A.m) {
    A.xs[off] = 0;
    A.xs[(size_t)K * A.npp + off] = 0;
    return;
  }
  const int row = 2 * n + h;
  float mx = -INFINITY;
  for (int s = 0; s < n_ranges; ++s)
    mx = fmaxf(mx, A.att[((size_t)(g * kFlashRanges + s) * ROWS + row) * (D + 2)]);
  float sum = 0.f, acc = 0.f;
  for (int s = 0; s < n_ranges; ++s) {
    const float* r = A.att + ((size_t)(g * kFlashRanges + s) * ROWS + row) * (D + 2);
    const float f = r[0] == -INFINITY ? 0.f : __expf(r[0] - mx);
    sum = fmaf(f, r[1], sum);
    acc = fmaf(f, r[2 + d], acc);
  }
  const float v = acc / sum;
  const uint16_t hb = to_bf16(v);
  A.xs[off] = hb;
  A.xs[(size_t)K * A.npp + off] = to_bf16(v - from_bf16(hb));
}

// ------------------------------------------------------------------ residual + norm
// grid (npp, H/512), 64 threads, 8 columns per thread: x[n] += the sum of the ks
// partials (in order); the layer output is recorded when slot >= 0; then gains * x
// split for the next product and the block's sum of squares.  KS > 0 is the partial count
// known at compile time: every partial's load is issued before the first add, so the
// thread waits for one memory round trip instead of one per few partials; KS = 0 reads
// the count from ks.
template <int KS>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 4))) void pf_resid_kernel(PfArgs A, const float* g,
                                                                                                int ks, int slot) {
  const int n = blockIdx.x, H = A.H, c = blockIdx.y * 64 + threadIdx.x;
  if (n >= A.m) { zero_split8(A.xs, H, A.npp, n, c); return; }
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, v[8];
  if constexpr (KS > 0) {
    float t[KS][8];
#pragma unroll
    for (int s = 0; s < KS; ++s) load8(A.part + ((size_t)s * A.npp + n) * H + 8 * c, t[s]);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] += t[s][e];
  } else {
#pragma unroll 8
    for (int s = 0; s < ks; ++s) {
      float t[8];
      load8(A.part + ((size_t)s * A.npp + n) * H + 8 * c, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] += t[e];
    }
  }
  float* x = A.x + (size_t)n * H + 8 * c;
  load8(x, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] += y[e];
  store8(x, v);
  if (slot >= 0 && A.dbg_hidden) store8(A.dbg_hidden + ((size_t)n * (A.L + 1) + slot) * H + 8 * c, v);
  gain_split(A, g, n, c, v);
}

// ------------------------------------------------------------------ SwiGLU
// grid (npp, I/256), 64 threads; thread t of block (n, b) takes the four intermediate
// columns 4(64b + t) .. +3.  Gate/up rows come in the arena's order: slice x of I/8
// columns, 32 runs of HALF = I/256 gate rows then HALF up rows; column c of the
// intermediate is gate row x*2IX + r*2HALF + i with x = c / IX, r = (c % IX) / HALF,
// i = c % HALF, and its up row HALF further.  HALF is a multiple of 4 (the host checks
// I % 1024), so a thread's four columns lie in one run and each partial is read as one
// float4 per half.  Both sums are scaled by the row's 1/rms (the post-attention norm).
// The output is split in natural column order, which is the down tiles' column order.
__global__ __launch_bounds__(64) void pf_swiglu_kernel(PfArgs A, int ks) {
  const int n = blockIdx.x, I = A.I, k0 = 4 * (blockIdx.y * 64 + threadIdx.x);
  // columns k0 .. k0+3 in the split layout: chunk k0/8, its half (k0 % 8) / 4
  const size_t off = ((size_t)(k0 / 8) * A.npp + n) * 8 + k0 % 8;
  uint2* hi = reinterpret_cast<uint2*>(A.xs + off);
  uint2* lo = reinterpret_cast<uint2*>(A.xs + (size_t)I * A.npp + off);
  if (n >= A.m) {
    *hi = make_uint2(0, 0);
    *lo = make_uint2(0, 0);
    return;
  }
  const int IX = I / kXcds, HALF = IX / kPerXcd, R = 2 * I;
  const float rs = row_rs(A, n);
  const int mg = (k0 / IX) * 2 * IX + ((k0 % IX) / HALF) * 2 * HALF + k0 % HALF;
  float gt[4] = {0.f, 0.f, 0.f, 0.f}, up[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = 0; s < ks; ++s) {
    const float* pp = A.part + ((size_t)s * A.npp + n) * R + mg;
    const float4 g4 = *reinterpret_cast<const float4*>(pp), u4 = *reinterpret_cast<const float4*>(pp + HALF);
    gt[0] += g4.x; gt[1] += g4.y; gt[2] += g4.z; gt[3] += g4.w;
    up[0] += u4.x; up[1] += u4.y; up[2] += u4.z; up[3] += u4.w;
  }
  uint32_t h[2], l[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    float v[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float gr = gt[2 * e + j] * rs;
      v[j] = gr / (1.f + __expf(-gr)) * (up[2 * e + j] * rs);
    }
    const uint16_t h0 = to_bf16(v[0]), h1 = to_bf16(v[1]);
    const uint16_t l0 = to_bf16(v[0] - from_bf16(h0)), l1 = to_bf16(v[1] - from_bf16(h1));
    h[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
  *hi = make_uint2(h[0], h[1]);
  *lo = make_uint2(l[0], l[1]);
}

// ------------------------------------------------------------------ first id
// Logits of the last prompt position: the final-norm row (gains * x * 1/rms) in LDS,
// 16 vocabulary rows per wave, 64 per workgroup, each row a 64-lane dot product over
// 16-byte weight loads; the workgroup's largest logit (ties: lowest row) goes to
// blk_val/blk_idx.  The row's sum of squares is taken from the row itself, so the
// kernel serves both prefill forms (only the residual row is common to them).  H is
// 1024 or 2048 here.
__global__ __launch_bounds__(256) void pf_lm_kernel(PfArgs A, LmArgs M) {
  constexpr int RPW = kLmRowsPerBlock / 4;
  __shared__ float xn[2048];
  __shared__ float bv[4];
  __shared__ int bi[4];
  __shared__ float sqw[4];
  const int H = A.H, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* x = A.x + (size_t)M.n_last * H;
  float sq = 0.f;
  for (int i = threadIdx.x; i < H; i += blockDim.x) sq = fmaf(x[i], x[i], sq);
  sq = wsum(sq);
  if (lane == 0) sqw[wv] = sq;
  __syncthreads();
  const float rs = rsqrtf((sqw[0] + sqw[1] + sqw[2] + sqw[3]) / (float)H + A.eps);
  for (int i = threadIdx.x; i < H; i += blockDim.x) xn[i] = M.g_final[i] * (x[i] * rs);
  __syncthreads();
  const int r0 = blockIdx.x * kLmRowsPerBlock + wv * RPW;
  float best = -INFINITY;
  int besti = 0x7fffffff;
  float acc[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) acc[j] = 0.f;
  for (int t = 0; t < H / 512; ++t) {  // 512 columns per pass, 8 per lane
    const int c = 8 * (lane + 64 * t);
    uint4 wr[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int r = min(r0 + j, A.vocab - 1);  // rows past the vocabulary re-read the last one
      wr[j] = *reinterpret_cast<const uint4*>(M.lm_head + (size_t)r * H + c);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const uint32_t w[4] = {wr[j].x, wr[j].y, wr[j].z, wr[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[j] = fmaf(__uint_as_float(w[e] << 16), xn[c + 2 * e], acc[j]);
        acc[j] = fmaf(__uint_as_float(w[e] & 0xffff0000u), xn[c + 2 * e + 1], acc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const float v = wsum(acc[j]);
    const int r = r0 + j;
    if (r < A.vocab && (v > best || (v == best && r < besti))) { best = v; besti = r; }
  }
  if (lane == 0) { bv[wv] = best; bi[wv] = besti; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int v = 1; v < 4; ++v)
      if (bv[v] > best || (bv[v] == best && bi[v] < besti)) { best = bv[v]; besti = bi[v]; }
    M.blk_val[blockIdx.x] = best;
    M.blk_idx[blockIdx.x] = besti;
  }
}

// The largest of the workgroup maxima (ties: lowest row), published: the device
// output, the feedback id, the pinned mirror, then the progress word.
__global__ __launch_bounds__(256) void pf_argmax_kernel(LmArgs M, int n_blk) {
  __shared__ float bv[256];
  __shared__ int bi[256];
  float best = -INFINITY;
  int besti = 0x7fffffff;
  for (int k = threadIdx.x; k < n_blk; k += blockDim.x) {
    const float v = M.blk_val[k];
    const int i = M.blk_idx[k];
    if (v > best || (v == best && i < besti)) { best = v; besti = i; }
  }
  bv[threadIdx.x] = best;
  bi[threadIdx.x] = besti;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      const float v = bv[threadIdx.x + s];
      const int i = bi[threadIdx.x + s];
      if (v > bv[threadIdx.x] || (v == bv[threadIdx.x] && i < bi[threadIdx.x])) {
        bv[threadIdx.x] = v;
        bi[threadIdx.x] = i;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int id = bi[0];
    if (id == 0x7fffffff) id = 0;  // every logit NaN: row 0
    M.out_first[0] = id;
    *M.last_id = id;
    if (M.pinned_ids)
      __hip_atomic_store(M.pinned_ids, ring_entry(M.call_seq, 0, id), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __threadfence_system();
    __hip_atomic_store(M.progress, ((unsigned long long)M.call_seq << 32) | 1ull, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// ------------------------------------------------------------------ self-test helpers
__global__ __launch_bounds__(64) void pf_split_kernel(const float* x, int K, int m, int npp, uint16_t* xs) {
  const int n = blockIdx.x;
  for (int c = threadIdx.x; c < K / 8; c += blockDim.x) {
    if (n >= m) { zero_split8(xs, K, npp, n, c); continue; }
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = x[(size_t)n * K + 8 * c + e];
    store_split8(xs, K, npp, n, c, v);
  }
}

__global__ __launch_bounds__(256) void pf_reduce_kernel(const float* part, int ks, int npp, int R, int m, float* y) {
  const int n = blockIdx.x;
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    float v = 0.f;
    for (int s = 0; s < ks; ++s) v += part[((size_t)s * npp + n) * R + r];
    y[(size_t)n * R + r] = v;
  }
}

// ------------------------------------------------------------------ host side
// How a product is cut: KC columns per wave (the widest of 256/128/64 dividing the K
// block that still gives 1024 waves or more: a wave streams 32 rows x KC columns, so
// narrower runs put more weight bytes in flight at once), and WK waves per workgroup
// over adjacent runs (the most, up to 4, whose WK*KC columns stay inside one K block),
// which leaves K / (WK*KC) partial sums per output.
struct Cut { int kc, wk, ks; };
Cut pick_cut(int R, int KB, int K) {
  Cut c{-1, 0, 0};
  if (R % 32 || KB % 64 || K % KB) return c;
  int kc = 256;
  while (kc > 64 && KB % kc) kc /= 2;
  while (kc > 64 && (R / 32) * (K / kc) < 1024) kc /= 2;
  int wk = 4;
  while (wk > 1 && KB % (wk * kc)) --wk;
  c.kc = kc;
  c.wk = wk;
  c.ks = K / (wk * kc);
  return c;
}

template <int NT>
int launch_gemm_nt(const uint16_t* w, int R, int KB, int K, Cut c, const uint16_t* xs, float* part, hipStream_t st) {
  const dim3 grid((R / 32) * c.ks), block(64 * c.wk);
  switch (c.kc) {
    case 64: hipLaunchKernelGGL((pf_gemm_kernel<NT, 1>), grid, block, 0, st, w, R, KB, K, xs, part); break;
    case 128: hipLaunchKernelGGL((pf_gemm_kernel<NT, 2>), grid, block, 0, st, w, R, KB, K, xs, part); break;
    case 256: hipLaunchKernelGGL((pf_gemm_kernel<NT, 4>), grid, block, 0, st, w, R, KB, K, xs, part); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemm(const uint16_t* w, int R, int KB, int K, int npp, const uint16_t* xs, float* part, hipStream_t st,
                int* ks) {
  const Cut c = pick_cut(R, KB, K);
  if (c.kc < 0) return -1;
  *ks = c.ks;
  switch (npp) {
    case 16: return launch_gemm_nt<1>(w, R, KB, K, c, xs, part, st);
    case 32: return launch_gemm_nt<2>(w, R, KB, K, c, xs, part, st);
    case 48: return launch_gemm_nt<3>(w, R, KB, K, c, xs, part, st);
    case 64: return launch_gemm_nt<4>(w, R, KB, K, c, xs, part, st);
  }
  return -1;
}

}  // namespace

size_t prefill_part_floats(int H, int NQ, int NKV, int D, int I) {
  const int QPG = NQ / NKV;
  const int dims[4][3] = {{NKV * (QPG + 2) * D, H, H}, {H, QPG * D, NQ * D}, {2 * I, H, H}, {H, I / kXcds, I}};
  size_t best = 0;
  for (const auto& d : dims) {
    const Cut c = pick_cut(d[0], d[1], d[2]);
    if (c.kc < 0) return 0;
    const size_t need = (size_t)c.ks * kPrefillChunk * d[0];
    if (need > best) best = need;
  }
  return best;
}

static void launch_resid(dim3 grid, hipStream_t st, const PfArgs& A, const float* g, int ks, int slot) {
  switch (ks) {
    case 8: hipLaunchKernelGGL(pf_resid_kernel<8>, grid, dim3(64), 0, st, A, g, ks, slot); break;
    case 16: hipLaunchKernelGGL(pf_resid_kernel<16>, grid, dim3(64), 0, st, A, g, ks, slot); break;
    default: hipLaunchKernelGGL(pf_resid_kernel<0>, grid, dim3(64), 0, st, A, g, ks, slot); break;
  }
}

int launch_prefill_chunk(const PfArgs& A, const uint8_t* layers, const LayerLayout& lay, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int H = A.H, D = A.D, NQ = A.NQ, NKV = A.NKV, I = A.I, QPG = NQ / NKV;
  if (D != 128 || QPG != 2 || H % 512 || I % 1024 || A.npp % 16 || A.npp > kPrefillChunk || A.m <= 0 || A.m > A.npp)
    return -1;
  const dim3 b256(256);
  const dim3 b64(64), rows_h(A.npp, H / 512), rows_i(A.npp, I / 256);
  hipLaunchKernelGGL(pf_input_kernel, rows_h, b64, 0, st, A);
  for (int l = 0; l < A.L; ++l) {
    const uint8_t* base = layers + (size_t)l * lay.stride;
    const float* G = reinterpret_cast<const float*>(base + lay.gains);
    int ks = 0;
    if (launch_gemm(reinterpret_cast<const uint16_t*>(base + lay.qkv), NKV * (QPG + 2) * D, H, H, A.npp, A.xs, A.part,
                    st, &ks))
      return -1;
    hipLaunchKernelGGL(pf_qkv_kernel, dim3(NKV, A.m), b256, 0, st, A, l, G, ks);
    if (A.pos0 + A.m <= kFlashMinKeys) {  // a short context: one workgroup per (group, position)
      hipLaunchKernelGGL(pf_attn_kernel, dim3(NKV, A.npp), dim3(64 * kPfAttnWaves), 0, st, A, l);
    } else {  // causal attention: key ranges on the matrix cores, then their merge
      const int kend = A.pos0 + A.m;
      int sk = kFlashKeys;
      while ((kend + sk - 1) / sk > kFlashRanges) sk += 32;
      const int nr = (kend + sk - 1) / sk;
      const dim3 fg(NKV, nr);
      switch (A.npp / 16) {
        case 1: hipLaunchKernelGGL(pf_flash_kernel<1>, fg, b256, 0, st, A, l, sk); break;
        case 2: hipLaunchKernelGGL(pf_flash_kernel<2>, fg, b256, 0, st, A, l, sk); break;
        case 3: hipLaunchKernelGGL(pf_flash_kernel<3>, fg, b256, 0, st, A, l, sk); break;
        default: hipLaunchKernelGGL(pf_flash_kernel<4>, fg, b256, 0, st, A, l, sk); break;
      }
      hipLaunchKernelGGL(pf_attn_combine_kernel, dim3(NKV, A.npp), b256, 0, st, A, nr);
    }
    if (launch_gemm(reinterpret_cast<const uint16_t*>(base + lay.o), H, QPG * D, NQ * D, A.npp, A.xs, A.part, st, &ks))
      return -1;
    launch_resid(rows_h, st, A, G, ks, -1);
    if (launch_gemm(reinterpret_cast<const uint16_t*>(base + lay.gu), 2 * I, H, H, A.npp, A.xs, A.part, st, &ks))
      return -1;
    hipLaunchKernelGGL(pf_swiglu_kernel, rows_i, b64, 0, st, A, ks);
    if (launch_gemm(reinterpret_cast<const uint16_t*>(base + lay.down), H, I / kXcds, I, A.npp, A.xs, A.part, st, &ks))
      return -1;
    launch_resid(rows_h, st, A, G + H + 2 * D, ks, l + 1);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_prefill_lm(const PfArgs& A, const LmArgs& M, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (A.H % 512 || A.H > 2048 || M.n_last < 0 || M.n_last >= A.m) return -1;
  const int n_blk = (A.vocab + kLmRowsPerBlock - 1) / kLmRowsPerBlock;
  hipLaunchKernelGGL(pf_lm_kernel, dim3(n_blk), dim3(256), 0, st, A, M);
  hipLaunchKernelGGL(pf_argmax_kernel, dim3(1), dim3(256), 0, st, M, n_blk);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemm_selftest(const uint16_t* w, int R, int K, const float* x, int m, float* y, uint16_t* xs, float* part,
                         void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int npp = (m + 15) / 16 * 16;
  hipLaunchKernelGGL(pf_split_kernel, dim3(npp), dim3(64), 0, st, x, K, m, npp, xs);
  int ks = 0;
  if (launch_gemm(w, R, K, K, npp, xs, part, st, &ks)) return -1;
  hipLaunchKernelGGL(pf_reduce_kernel, dim3(m), dim3(256), 0, st, part, ks, npp, R, m, y);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mk
