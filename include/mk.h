/*
 * mk.h -- C ABI of the persistent-megakernel batch-1 decoder for AMD MI355X (gfx950).
 *
 * The library runs the autoregressive decode step of a Qwen3-style decoder (the
 * talker of a streaming TTS model) as ONE persistent kernel that loops over decode
 * steps inside the kernel, instead of launching one kernel per operation:
 *   - dev.to, "Porting a 1,200-line persistent CUDA megakernel to Qwen3-TTS",
 *     section "The idea: one kernel that never exits": a decode step is embedding
 *     lookup, attention, MLP, norms and sampling; the persistent kernel owns the GPU
 *     and loops over steps itself.
 *   - same article, "Porting it to Qwen3-TTS-1.7B": untied embeddings (the LM head
 *     reads its own matrix) and multi-section rotary embeddings.
 *   - theaicatchup, "I made a single CUDA kernel speak", section "Why Does a Single
 *     Kernel Even Matter for TTS?": the talker body equals Qwen3-0.6B; its inputs are
 *     sums of 17 embeddings, handed over through a sentinel: an id >= 0 is a table
 *     lookup, an id < 0 means "take the precomputed row".
 *   - same article, "So, What's the Catch with These Megakernels?": rotary
 *     frequency tables are built on the host.
 *
 * Conventions shared by every entry point
 *   - Pointers named d_* are DEVICE pointers (e.g. from torch tensors on the GPU);
 *     h_* are host pointers.  The library borrows them for the stream-ordered
 *     duration of the call and never frees them.
 *   - Matrices are row-major [out][in] (the HF layout).  bf16 tensors are raw
 *     16-bit patterns; f32 tensors are IEEE float.
 *   - Every call is asynchronous on the handle's stream unless stated otherwise.
 *     Argument errors are detected on the host before anything is launched and
 *     returned as a negative code; faults found on the device (an id outside the
 *     vocabulary, a wait that timed out) are latched in a device error word and
 *     reported by the next mk_status().
 *   - A handle is bound to one device and one stream and is not thread-safe.
 */
#ifndef MK_H
#define MK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------------- */
#define MK_OK               0
#define MK_ERR_ARG         -1   /* null pointer, bad size, bad cfg field            */
#define MK_ERR_UNSUPPORTED -2   /* cfg is valid but no kernel body is built for it  */
#define MK_ERR_OOM         -3   /* device or pinned allocation failed               */
#define MK_ERR_CAPACITY    -4   /* position + n would exceed cfg.max_seq            */
#define MK_ERR_COOP        -5   /* one workgroup per CU cannot be made co-resident  */
#define MK_ERR_HIP         -6   /* a HIP runtime call failed                        */
#define MK_ERR_DEVICE      -7   /* device error word: bad id or bad position        */
#define MK_ERR_TIMEOUT     -8   /* device error word: a cross-workgroup wait timed out */
#define MK_ERR_STATE       -9   /* call order: e.g. feedback decode with no previous id */
#define MK_ERR_SCRATCH    -10   /* the shape needs more than MK_STATIC_SCRATCH_BYTES of scratch */
#define MK_ERR_OVERRUN    -11   /* the id ring moved past ids not yet read            */

/* Entries of the pinned id ring that mk_read_ids reads (4096). */
#define MK_ID_RING 4096

/* Size of the fixed device array mk_prefill_batched_noalloc works in (48 MiB); every
 * device the library runs on holds one from its first handle until the process ends. */
#define MK_STATIC_SCRATCH_BYTES (48u << 20)

/* ---- dtypes ----------------------------------------------------------------- */
#define MK_F32  0
#define MK_BF16 1

/* Model configuration.  Body shapes with a compiled kernel:
 *   hidden 256,  head_dim 64,  16/8 -> 4/2 heads, intermediate 768,  f32 weights  (tiny)
 *   hidden 1024, head_dim 128, 16 q / 8 kv heads, intermediate 3072, bf16 weights (Qwen3-0.6B body)
 *   hidden 2048, head_dim 128, 16 q / 8 kv heads, intermediate 6144, bf16 weights (1.7B-scale talker)
 * The KV cache is kept in the body's weight dtype (kv_dtype must equal weight_dtype).
 * n_layers, vocab (< 2^18), max_seq, tied, rms_eps, rope_theta and the rotary
 * sections are free.  sections[0..n_sections) are counts of rotary PAIRS, contiguous
 * from pair 0, summing to head_dim/2; section k turns with position stream k
 * ({head_dim/2} with n_sections = 1 is ordinary RoPE). */
typedef struct mk_cfg {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab;
  int32_t tied;          /* 1: the LM head reads the input embedding matrix          */
  int32_t weight_dtype;  /* MK_F32 | MK_BF16 (every weight tensor, gains included)   */
  int32_t kv_dtype;      /* MK_F32 | MK_BF16: KV cache storage; bf16 rounds to nearest even */
  float   rms_eps, rope_theta;
  int32_t n_sections, sections[3];
  int32_t max_seq;       /* KV capacity in positions                                 */
} mk_cfg;

/* Weights, all device pointers, HF layout.  Per-layer entries are HOST arrays of
 * n_layers device pointers.  Shapes: embed [vocab][hidden]; lm_head [vocab][hidden]
 * (NULL when tied); final_norm, in_norm, post_norm [hidden]; wq [n_q*d][hidden];
 * wk, wv [n_kv*d][hidden]; q_norm, k_norm [d]; wo [hidden][n_q*d];
 * w_gate, w_up [intermediate][hidden]; w_down [hidden][intermediate].
 * mk_create copies everything into a library-owned arena; the caller may free its
 * tensors once mk_create has returned (it synchronizes the stream). */
typedef struct mk_weights {
  const void *embed, *lm_head, *final_norm;
  const void *const *in_norm, *const *wq, *const *wk, *const *wv, *const *q_norm, *const *k_norm,
             *const *wo, *const *post_norm, *const *w_gate, *const *w_up, *const *w_down;
} mk_weights;

typedef struct mk_handle mk_handle;

/* Build a decoder: the dev.to article "Porting a 1,200-line persistent CUDA megakernel to
 * Qwen3-TTS", "Porting it to Qwen3-TTS-1.7B", fixes the model constants when the decoder is
 * built (vocabulary, untied head, rotary sections), and the theaicatchup article, "So,
 * What's the Catch with These Megakernels?", has the rotary frequency tables computed on
 * the host; both are what this call does before any decode.
 * Validate cfg, allocate the arena, KV cache, exchange buffers, the pinned
 * progress word and the pinned id ring (MK_ID_RING entries, reused by every call: no
 * call ever grows it), pack the weights, build the rotary cos/sin table (computed in
 * double, stored as float) and check that one workgroup per CU fits co-resident.
 * MK_ERR_ARG if max_seq >= 2^26 (the ring's entries number slots below that).
 * The first handle on a device also looks up that device's address of the fixed
 * scratch array of mk_prefill_batched_noalloc (MK_ERR_HIP if that fails).
 * stream: a hipStream_t (NULL = the null stream).  Synchronous.
 * Returns MK_OK and *out, or a negative code with *out = NULL. */
int mk_create(const mk_weights* w, const mk_cfg* cfg, void* stream, mk_handle** out);

/* The prompt before the first decode step (dev.to article, "Making it talk end-to-end":
 * the first audio chunk waits for the prompt, so it is part of the time to first chunk).
 * Run n prompt positions starting at the current position (0 after create/reset,
 * n_pos after mk_load_kv) position by position through the same persistent kernel;
 * the LM head runs only at the last one and its greedy id (ties: lowest index) is
 * written to d_out_first[0] (device int32) and kept as the feedback id.
 *   d_ids  [n] int32: >= 0 reads embed[id]; < 0 reads row t of d_rows.
 *   d_rows [n][hidden] float32, may be NULL when no id is negative.
 *   d_pos3 [n][3] int32 rotary position streams, or NULL: every stream = position.
 * MK_ERR_CAPACITY if position + n > max_seq. */
int mk_prefill(mk_handle* h, const int32_t* d_ids, const float* d_rows, const int32_t* d_pos3,
               int32_t n, int32_t* d_out_first);

/* Same contract and arguments as mk_prefill, with the prompt run as a batch: up to 64
 * positions per pass over the weights (matrix-core products over the packed weight
 * tiles, causal attention over the cache, the cache written as mk_prefill writes it),
 * then the LM head over the last position and its greedy id (ties: lowest index),
 * published as mk_prefill publishes it (d_out_first[0], the feedback id, the pinned id
 * ring and the progress word).  A chunk of positions runs in one of two forms (see
 * mk_set_prefill_path): one persistent launch for all layers, whose phases hand over
 * through flagged buffers (hidden 1024 with intermediate 3072, contexts up to 2048
 * positions), or a chain of ordinary per-layer kernels (every supported shape).  The time to the first id is where per-position work costs most
 * (the dev.to article "Porting a 1200-line persistent CUDA megakernel to Qwen3-TTS",
 * "Making it talk end-to-end"), and a batch is the case a one-position-per-pass
 * persistent loop does not serve well (same article, "What I took away").  Results
 * equal mk_prefill's up to rounding order, the debug hidden states too; the barrier
 * trace and phase timeline are not written for these positions.
 * Allocates its scratch (about 40 MB at hidden 2048) on the first call.
 * MK_ERR_UNSUPPORTED for float32 weights, a hidden size that is not a multiple of 512,
 * an intermediate size that is not a multiple of 1024, hidden above 2048, or a head layout other than head_dim 128 with
 * two query heads per KV head (use mk_prefill there); other errors as mk_prefill.
 * Stream-ordered on the handle's stream; an id or position outside its table is
 * flagged in the device error word and read as 0, as in mk_prefill. */
int mk_prefill_batched(mk_handle* h, const int32_t* d_ids, const float* d_rows, const int32_t* d_pos3,
                       int32_t n, int32_t* d_out_first);

/* mk_prefill_batched for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * kernels and results (bit for bit) as mk_prefill_batched; its scratch is a fixed
 * array of MK_STATIC_SCRATCH_BYTES per device instead of a buffer the handle allocates,
 * and it calls no allocating routine (the pinned ring entry it publishes into was
 * allocated by mk_create).  Every call on a device shares that device's array and
 * leaves its contents behind; each word a call reads it has written first, so nothing
 * needs clearing.  Calls that overlap on one device, from any handle or stream, race
 * on the array: the caller orders them.  MK_ERR_SCRATCH if the handle's shape needs
 * more than the array holds (no shape with a built body does: the hidden-2048 body
 * needs about 41 MiB, whatever n is, as the prompt runs in chunks of 64); MK_ERR_STATE
 * if the array's device address is not known (mk_create looks it up on the handle's
 * device); other errors as mk_prefill_batched. */
int mk_prefill_batched_noalloc(mk_handle* h, const int32_t* d_ids, const float* d_rows, const int32_t* d_pos3,
                               int32_t n, int32_t* d_out_first);

/* The hot path: n_steps decode steps in ONE launch.  Step s runs at position
 * position+s and reads
 *   d_ids == NULL : the id picked by the previous step (step 0: by the last prefill
 *                   or decode call; MK_ERR_STATE if there is none): embed[id], and
 *                   when d_embed_buf is given, embed[id] + row s of d_embed_buf: the
 *                   talker's fed-back codebook-0 embedding plus the rest of the frame's
 *                   17 embeddings, summed by the caller (the theaicatchup article, "Why
 *                   Does a Single Kernel Even Matter for TTS?": the input is a sum of
 *                   16 codebook embeddings and a text embedding);
 *   d_ids[s] >= 0 : embed[d_ids[s]];
 *   d_ids[s] <  0 : row s of d_embed_buf ([n_steps][hidden] float32).
 * d_pos3 as in mk_prefill.  d_out_ids [n_steps] int32 receives the greedy ids
 * (ties: lowest index); each id also goes to the pinned id ring (see mk_read_ids) and
 * the pinned progress word advances after every step. */
int mk_decode(mk_handle* h, int32_t n_steps, const int32_t* d_ids, const float* d_embed_buf,
              const int32_t* d_pos3, int32_t* d_out_ids);

/* The launch tax, measured (the dev.to article "Porting a 1,200-line persistent CUDA
 * megakernel to Qwen3-TTS", "What I took away": every kernel launch of a step costs
 * latency; the theaicatchup article, "Why Does a Single Kernel Even Matter for TTS?":
 * a normal forward pass launches hundreds of kernels).  mk_decode's computation with
 * the persistent kernel's own phase bodies (same grid, tiles, LDS copies, arithmetic
 * and exchange buffers), but one kernel launch per phase: 7 per layer and one for the
 * LM head per step (197 at 28 layers), each launch reading the words the one before
 * published.  Same arguments and results as mk_decode, bit for bit (ids, cache,
 * hidden states); the barrier trace and phase timeline are not written.  Measurement
 * only.  MK_ERR_UNSUPPORTED for any body other than the hidden-1024 bf16 one; other
 * errors as mk_decode.  Stream-ordered on the handle's stream. */
int mk_decode_phased(mk_handle* h, int32_t n_steps, const int32_t* d_ids, const float* d_embed_buf,
                     const int32_t* d_pos3, int32_t* d_out_ids);

/* A cache that already holds n_pos positions: the conversation history a later decode
 * attends over (the dev.to article, "The idea: one kernel that never exits": attention at
 * each step reads every cached position; the long-context workloads start from such a
 * cache).  Install n_pos already-rotated cache positions and set the position to n_pos.
 * d_kv: device [n_layers][2][n_kv][n_pos][head_dim] in cfg.kv_dtype (K then V), copied
 * stream-ordered (the caller may free it after the stream reaches this point).
 * MK_ERR_ARG for a NULL handle or pointer or n_pos < 0; MK_ERR_CAPACITY if n_pos > max_seq. */
int mk_load_kv(mk_handle* h, const void* d_kv, int32_t n_pos);

/* Start a new utterance on the same decoder (the dev.to article, "Making it talk
 * end-to-end": each utterance is its own prompt and decode).  Rewind to position 0 and
 * forget the feedback id (the cache is not cleared: it is only read at positions that
 * have been written since), and re-arm the device side, stream-ordered: the device error
 * word, the abort flag a timed-out wait raised and the timeout record are cleared.  Read
 * them first with mk_status / mk_error_info if they matter.  MK_ERR_ARG for a NULL handle,
 * MK_ERR_HIP if the clearing cannot be enqueued. */
int mk_reset(mk_handle* h);

/* Current position (positions written so far).  Host only, no sync. */
int mk_position(mk_handle* h, int32_t* pos);

/* Debug outputs of the following prefill/decode calls (NULL turns each off):
 *   d_hidden [n][n_layers+1][hidden] float32: the residual stream entering layer 0
 *            and leaving every layer, for each position the call runs;
 *   d_trace  [n][grid][2] uint64: per position and workgroup, the 100 MHz ticks spent
 *            waiting for other workgroups and the ticks of the whole position. */
int mk_set_debug(mk_handle* h, float* d_hidden, uint64_t* d_trace);

/* Barrier timeline of one workgroup for the following prefill/decode calls (NULL
 * turns it off): d_phase [n][2 + 10*n_layers][8] uint64 receives, for each position
 * the call runs and each workgroup barrier of that position in program order (input
 * fetch, ten per layer, LM head), the 100 MHz ticks at which workgroup wg's control
 * wave arrived at it and left it, then the ticks at which the first two waits for
 * other workgroups' words in the segment before that barrier completed, then (first
 * worker wave) when it had issued its weight copies, finished its dot product and
 * arrived at the barrier, and last, for the first wait of the segment, its poll rounds
 * (bits 56..63), the ticks of its first round (bits 32..55) and all its ticks (bits
 * 0..31) (0 where an event does not occur).  wg = -1 traces every
 * workgroup: d_phase is then [n][grid][2 + 10*n_layers][8].  The persistent form of
 * mk_prefill_batched writes instead, for each chunk it runs (each overwriting the one
 * before), [grid][n_layers + 1][8][2]: for each hand-over kind (q/k/v, attention, O
 * partials, residual after attention, SwiGLU, down partials, residual after the MLP,
 * and in slot 0 the launch's placement check) produced in layer l (slot l + 1; slot 0
 * also holds the input rows' residual), the 100 MHz ticks at which the workgroup's wait
 * for it completed and at which the workgroup raised its own flag of that kind.
 * MK_ERR_ARG if wg is not in [-1, grid). */
int mk_set_phase_trace(mk_handle* h, uint64_t* d_phase, int32_t wg);

/* Which form mk_prefill_batched and mk_prefill_batched_noalloc run a call in:
 *   MK_PREFILL_AUTO        the persistent form where the call has it, else the chain;
 *   MK_PREFILL_CHAIN       the per-layer kernel chain;
 *   MK_PREFILL_PERSISTENT  the persistent form; calls without it (another shape, or a
 *                          context past 2048 positions) return MK_ERR_UNSUPPORTED.
 * Both forms compute the same sums in different rounding orders.  MK_ERR_ARG for a NULL
 * handle or another value. */
#define MK_PREFILL_AUTO 0
#define MK_PREFILL_CHAIN 1
#define MK_PREFILL_PERSISTENT 2
int mk_set_prefill_path(mk_handle* h, int32_t path);

/* Poll rounds after which a wait for other workgroups' words gives up, for the following
 * prefill/decode calls (polls == 0 restores the default, 2^22, about a second).  A wait
 * that gives up latches MK_ERR_TIMEOUT in the device error word and raises the abort
 * flag; every other wait sees the flag within 128 rounds, so every wave of the launch
 * leaves and the call completes; mk_status then returns MK_ERR_TIMEOUT, mk_error_info
 * says where, and mk_reset (which clears the flag and the error word) re-arms the handle.  A small limit is
 * how a host forces that path.  MK_ERR_ARG for a NULL handle. */
int mk_set_spin_limit(mk_handle* h, uint32_t polls);

/* Ids published so far by the most recently enqueued prefill/decode call (0 until
 * its first id), read from pinned host memory without synchronizing: the basis of
 * time-to-first-chunk.  A prefill publishes one id. */
int mk_progress(mk_handle* h, int64_t* steps_done);

/* Host-side streaming of the ids as they are published (the dev.to article "Porting a
 * 1200-line persistent CUDA megakernel to Qwen3-TTS", "Making it talk end-to-end":
 * audio tokens leave chunk by chunk, and the first chunk cannot wait for the rest).
 * Copies ids [first, first + count) of the most recently enqueued
 * prefill/decode call from the pinned id ring into host_out, without synchronizing.
 * The ring holds MK_ID_RING entries: id s of a call goes to entry s % MK_ID_RING,
 * tagged with its call and its lap s / MK_ID_RING, so a call of any length streams
 * through it with no synchronization, as long as the reader stays fewer than
 * MK_ID_RING ids behind the kernel.  An entry the progress word already counts but
 * that has not arrived yet (the device does not order the two stores) is read again
 * until it does.  MK_ERR_ARG if fewer than first + count ids are published yet (see
 * mk_progress) or an argument is out of range; MK_ERR_OVERRUN if a later lap has
 * already overwritten an entry asked for (the ids stay in the call's d_out_ids);
 * MK_ERR_TIMEOUT if a counted entry never arrives. */
int mk_read_ids(mk_handle* h, int32_t first, int32_t count, int32_t* host_out);

/* *idle = 1 if the handle's stream has finished everything enqueued on it, else 0;
 * no synchronization (a poll loop over mk_progress uses it to notice a call that
 * ended early, e.g. on a wait timeout).  MK_ERR_HIP if the stream reports an error. */
int mk_query(mk_handle* h, int32_t* idle);

/* Faults found inside the running kernel (an id outside the vocabulary, a position
 * outside the rotary table, a wait for another workgroup that gave up) cannot return
 * from a launch that loops over many steps (the dev.to article, "The idea: one kernel
 * that never exits"): they are latched on the device and read here.
 * Synchronize the stream and report the device error word: MK_OK when clean,
 * MK_ERR_TIMEOUT after a wait gave up, MK_ERR_DEVICE for a bad id or position,
 * MK_ERR_HIP if the stream reports an error.  The word and the abort flag are cleared
 * by the read. */
int mk_status(mk_handle* h);

/* Where the first wait that timed out was (after mk_status returned MK_ERR_TIMEOUT):
 * info[0] = 1 if recorded, then the workgroup, the tag it waited for, the word offset
 * of that word from the start of the handle's exchange buffers, and the tag found
 * there.  Synchronizes the stream; reading re-arms the record. */
int mk_error_info(mk_handle* h, int32_t* info /* [5] */);

/* Self-test of the LDS DMA copy the kernel streams weights with: one workgroup copies
 * n_chunks 16-byte chunks of d_src into LDS at byte offset offset_bytes, then back out to
 * d_dst (device buffers of n_chunks * 16 bytes).  offset_bytes + 16 n_chunks <= 147456. */
int mk_selftest_lds_dma(const void* d_src, void* d_dst, int32_t n_chunks, int32_t offset_bytes, void* stream);

/* Self-test of the batched prefill's matrix product: d_y[t][r] = sum over k of
 * d_w[r][k] * d_x[t][k], d_w [rows][k] bf16, d_x [n][k] float32, d_y [n][rows] float32,
 * through the same activation split and MFMA product kernels.  rows % 32 == 0,
 * k % 64 == 0, 1 <= n <= 64, else MK_ERR_ARG.  Allocates and frees its scratch;
 * synchronizes `stream`. */
int mk_selftest_gemm(const void* d_w, int32_t rows, int32_t k, const float* d_x, int32_t n, float* d_y,
                     void* stream);

/* Measurement kernel: one streaming read of `bytes` from d_src (16-byte loads, 256
 * threads per workgroup, `blocks` workgroups in a grid-stride loop; non-temporal
 * loads when nontemporal != 0).  Its time gives the read bandwidth the device
 * reaches, the ceiling the decode kernel's achieved bytes per second compare with.
 * d_sink [blocks] uint64 is written only in a case that does not occur for real
 * data patterns, so the loads stay.  Asynchronous on `stream`.  MK_ERR_ARG for NULL
 * pointers, bytes not a positive multiple of 16, or blocks outside 1..65536. */
int mk_bench_stream_read(const void* d_src, uint64_t bytes, int32_t nontemporal, uint64_t* d_sink, int32_t blocks,
                         void* stream);

/* Stress test of the tagged-word exchange every hop of the decode kernel uses (its own
 * publish and gather code): one cooperative launch of the persistent grid runs `iters`
 * rounds; in each, every workgroup publishes 64 words and gathers the round's words of
 * its partners, checking every value against what its writer stored.
 *   xcd_local == 0: all to all (256 x 64 words a round), every word written through to
 *                   the device coherence point: the decode kernel's cross-XCD hops;
 *   xcd_local != 0: each workgroup with the 32 of its XCD (workgroups b with the same
 *                   b % 8; 32 x 64 words a round), and, when a placement check finds
 *                   every workgroup b on XCD b % 8, with plain stores that stay in that
 *                   XCD's L2: the decode kernel's local hops.
 * result (host, [4]): [0] words read with the right tag but a wrong value (stale or
 * torn: must be 0), [1] workgroups whose wait gave up, [2] the device error word, [3] 1
 * if the plain stores were used (xcd_local only).  spin_limit as in mk_set_spin_limit
 * (0: the default); a small limit forces the give-up path.  Allocates and frees its
 * buffers; synchronizes `stream`.  MK_ERR_ARG for iters <= 0 or a NULL result;
 * MK_ERR_COOP if the grid cannot be launched co-resident. */
int mk_selftest_exchange(int32_t iters, uint32_t spin_limit, int32_t xcd_local, uint32_t* result, void* stream);

/* Number of workgroups of the persistent grid (one per CU). */
int mk_grid_size(mk_handle* h, int32_t* n);

/* Talker input rows on the device: row t = sum over c of codebooks[c][ids[t][c]]
 * (c = 0..n_codebooks-1) plus text[ids[t][n_codebooks]], widened to float32 and
 * added one row at a time in that order (the theaicatchup article, "Why Does a
 * Single Kernel Even Matter for TTS?": inputs are sums of 16 codebook embeddings
 * and a text embedding).
 *   d_codebooks [n_codebooks][codebook_size][hidden], d_text [text_vocab][hidden],
 *   both in dtype (MK_F32 | MK_BF16); d_ids [n][n_codebooks+1] int32;
 *   d_rows [n][hidden] float32 (output).  An id outside its table reads row 0 of
 *   that table and adds one to d_bad[0] (device int32) when d_bad is not NULL.
 *   n == 0 does nothing (the pointers may then be NULL).  MK_ERR_ARG for a negative
 *   n, a non-positive size, an unknown dtype or a NULL pointer with n > 0.
 *   Stream-ordered on `stream` (a hipStream_t, NULL = null stream). */
int mk_embed_sum(const void* d_codebooks, int32_t n_codebooks, int32_t codebook_size,
                 const void* d_text, int32_t text_vocab, int32_t hidden, int32_t dtype,
                 const int32_t* d_ids, int32_t n, float* d_rows, int32_t* d_bad, void* stream);

const char* mk_strerror(int code);

/* Free everything the handle owns.  Synchronizes its stream.  NULL is a no-op. */
void mk_destroy(mk_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
