/*
 * lsh_attn.h -- C ABI of the LSH-sampled decode-attention library (gfx950).
 *
 * MagicPIG replaces the attention of a decode query by an estimate built from
 * keys sampled with locality-sensitive hashing ("MagicPIG: LSH Sampling for
 * Efficient LLM Generation", GrooveSquid summary; MagicPIG project summary on
 * sourcepulse, "How It Works"), behind an LSH library that exposes an LSH
 * kernel through an interface header ("How infini-ai-lab/magicpig works",
 * Components: "LSH Sampling").  This header is that interface for MI355X.
 * The library has two operations:
 *
 *   lsh_build_tables      at prefill: SimHash every key into L codes of K bits
 *                         and bucket the keys of every table (the hash-table
 *                         construction the sourcepulse summary lists under
 *                         "Highlighted Details").
 *   lsh_decode_attention  at a decode step: hash each query head, probe its L
 *                         buckets, count per-key collisions, keep keys that
 *                         collide in >= T tables, and return the 1/u-weighted
 *                         softmax estimate and its log-sum-exp.
 *
 * Definitions (d = head dim, N = keys per sequence, G = Hq / Hkv):
 *   proj      = k @ W, W of shape [d, L*K]; column l*K + b is bit b of table l.
 *   code_l(k) = sum_b [proj[l*K + b] > 0] << b        (bit 0 = LSB, 0 -> bit 0)
 *   c(n)      = #{ l : code_l(k_n) == code_l(q) }      (collision count)
 *   S         = { n : c(n) >= T }                       (selected keys)
 *   P(n)      = (1 - theta_n / pi)^K, theta_n the angle between q and k_n
 *               (cos := 0 when a norm is 0)
 *   u(n)      = P[Binomial(L, P(n)) >= T], clamped to >= 1e-30
 *   l(n)      = sm_scale * q.k_n - ln u(n)
 *   out       = sum_{n in S} softmax(l)_n v_n,  lse = ln sum_{n in S} exp l(n)
 *               (S empty: out = 0, lse = -inf)
 *   Query head h reads kv head h / G.
 *
 * Conventions for every entry point:
 *   - Every pointer argument is DEVICE memory owned by the caller, except
 *     `stream`, which is a hipStream_t handle (NULL = the null stream).  The
 *     library allocates no device memory of its own at run time; the state it
 *     keeps between calls is host-side bookkeeping that never changes a
 *     result: the kernel-timing window at the end of this header, the record
 *     of which kernels already had their LDS limit raised on which device, and
 *     the per-device address of the static scratch array that
 *     lsh_decode_attention_noalloc uses (the library's one device-side state,
 *     loaded with the code object).  Calls on different streams may run
 *     concurrently if they use separate outputs and workspaces.
 *   - All arrays are dense, row-major (last index fastest), 16-byte aligned.
 *   - Work is enqueued on `stream` and the call returns without waiting.
 *     The returned status covers argument checks (made before anything is
 *     enqueued; on error nothing is launched and no output is touched) and
 *     launch errors; a fault during execution shows at the caller's next
 *     synchronisation.
 *   - Required outputs are fully written.  Optional outputs (may be NULL) are
 *     written only when non-NULL.
 *   - dtype: LSH_BF16 or LSH_F32, the element type of keys, values, q and W.
 *     Projections and dot products accumulate in fp32; outputs are fp32.
 */
#ifndef LSH_ATTN_H
#define LSH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LSH_OK = 0,
  LSH_ERR_INVALID_ARG = 1,  /* null required pointer, bad size or parameter */
  LSH_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. d != 128)   */
  LSH_ERR_WORKSPACE = 3,    /* workspace_bytes below the size query        */
  LSH_ERR_HIP = 4           /* a HIP runtime call or launch failed          */
} lsh_status;

typedef enum { LSH_F32 = 0, LSH_BF16 = 1 } lsh_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* lsh_status_string(int status);

/* Number of key chunks of a table: ceil(N / stride). */
int lsh_num_chunks(int N, int stride);

/* A chunk stride for N keys and K bits: the smallest power of two >= 256 and
 * >= N, capped at 8192.  Any valid stride describes the same buckets; the
 * stride sets how the keys are split into chunks, each sorted on its own.
 * Returns 0 for N < 1 or K outside 0..15. */
int lsh_default_stride(int N, int K);

/* ------------------------------------------------------------------------
 * Table build
 *
 * Size limits: B, Hkv, N >= 1; d == 128 (else LSH_ERR_UNSUPPORTED);
 * 0 <= K <= 15; 1 <= L <= 255; stride a power of two in [256, 8192]
 * (else LSH_ERR_UNSUPPORTED); N <= 2^30, B*Hkv*L*N < 2^40 and B*Hkv*L < 2^31
 * (else LSH_ERR_UNSUPPORTED).
 *
 * Layout of the tables (two-level CSR, chunk-major).  The keys of a table are
 * cut into nchunks = lsh_num_chunks(N, stride) chunks of `stride` keys (the
 * last one ragged); chunk j holds keys j*stride .. min(N, (j+1)*stride) - 1 and
 * owns positions j*stride .. of indices[b,g,l,:].  Inside its region a chunk
 * lists its keys grouped by bucket in ascending code order, ascending key index
 * inside each bucket, each entry holding (key index - j*stride).  Bucket c of
 * chunk j therefore occupies region positions offsets[b,g,l,j,c] ..
 * offsets[b,g,l,j,c+1] (for c = 2^K - 1: .. the chunk's length).  Bucket c of
 * the whole table is the concatenation over j of these segments.
 * ---------------------------------------------------------------------- */

/* Bytes of device workspace lsh_build_tables needs (0 on invalid sizes). */
size_t lsh_build_workspace_size(int B, int Hkv, int N, int d, int K, int L,
                                int stride, int dtype);

/*
 * keys     [B, Hkv, N, d]  dtype        key cache of every (sequence, kv head)
 * W        [d, L*K]        dtype        SimHash projection, shared by all heads
 * offsets  [B, Hkv, L, nchunks, 2^K] uint16
 *                                       out: start of bucket c inside chunk j's
 *                                       region (see the layout above)
 * indices  [B, Hkv, L, N]  uint16       out: chunk-relative key indices, grouped
 *                                       by chunk, then bucket, then key
 * key_codes [B, Hkv, L, N] uint16       optional out: code_l(k_n)
 * workspace                             device scratch of the queried size
 */
lsh_status lsh_build_tables(const void* keys, const void* W,
                            int B, int Hkv, int N, int d, int K, int L,
                            int stride, int dtype,
                            uint16_t* offsets, uint16_t* indices,
                            uint16_t* key_codes,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Table update for a growing key cache.  The pages build the tables once
 * over the prompt (sourcepulse summary, "Highlighted Details": hash-table
 * construction) and say nothing of the keys a decode appends; MAC-Attention
 * updates its caches for the next token inside the decode step
 * ("MAC-Attention" README, "How It Works").  Here the tables of a cache with
 * room for n_cap keys per (sequence, kv head) hold its first n_b keys
 * (sequence b), and
 *
 *   after lsh_update_tables, the tables of sequence b are exactly those that
 *   lsh_build_tables would produce from its keys 0 .. new_b - 1
 *
 * (same codes, buckets, order and offsets), laid out with the pitch n_cap:
 *
 * keys     [B, Hkv, n_cap, d] dtype     keys 0 .. new_b - 1 written
 * W        [d, L*K], or [Hkv, d, L*K] with w_per_head = 1 (kv head g hashes
 *          with W[g]; queries of head h with W[h / G])
 * offsets  [B, Hkv, L, lsh_num_chunks(n_cap, stride), 2^K] uint16
 *                                       in/out: chunks j < old_b / stride are
 *                                       kept; the rest up to new_b rewritten
 * indices  [B, Hkv, L, n_cap] uint16    in/out: positions below
 *                                       (old_b / stride) * stride are kept
 * key_codes [B, Hkv, L, n_cap] uint16   optional out: codes of keys old_b ..
 *                                       new_b - 1 (of the keys from
 *                                       (old_b / stride) * stride when the
 *                                       chunks are rebuilt, below)
 * old_lens, new_lens [B] int32          optional (device): old_b, new_b per
 *                                       sequence; when NULL every old_b =
 *                                       n_old, every new_b = n_new
 * workspace                             lsh_build_workspace_size(.., n_cap, ..)
 *
 * (x / stride rounds down.)  The inputs must hold the tables of exactly the
 * keys 0 .. old_b - 1, built with the same W, K, L, stride and n_cap
 * (old_b = 0: nothing); keys of positions >= new_b are never read.  A
 * sequence that gains at most 256 keys onto tables holding some (old_b > 0,
 * new_b - old_b <= 256) has them inserted: only the new keys are projected,
 * and in the one or two chunks they fall into the entries after each
 * insertion point move up and the bucket starts are raised.  Any other
 * sequence has the chunks from the one holding key old_b to the one holding
 * key new_b - 1 rebuilt from their keys.  The scalars bound the arrays:
 * n_old <= old_b <= new_b <= n_new, with device values clamped into that
 * range (the launch covers the chunks of keys n_old .. n_new - 1).  Each
 * sequence's choice is taken on the device from its own lengths; the host
 * leaves the rebuild kernels out only when the bounds settle it for every
 * sequence (0 < n_old, n_new - n_old <= 256), so a step captured in a graph
 * with bounds that close runs the insertion alone, and one with wider bounds
 * also launches the rebuild kernels, whose workgroups then return at once
 * for the sequences that insert.  0 <= n_old <= n_new <= n_cap and
 * w_per_head in {0, 1}, else LSH_ERR_INVALID_ARG; n_old == n_new launches
 * nothing.  Size limits as for lsh_build_tables with N = n_cap.
 * lsh_build_tables(.., N, ..) is this call with n_old = 0, n_new = n_cap = N,
 * no length arrays and a shared W.
 */
lsh_status lsh_update_tables(const void* keys, const void* W,
                             int B, int Hkv, int n_old, int n_new, int n_cap,
                             const int32_t* old_lens, const int32_t* new_lens,
                             int d, int K, int L, int stride, int dtype,
                             int w_per_head,
                             uint16_t* offsets, uint16_t* indices,
                             uint16_t* key_codes,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * Decode
 *
 * Size limits: those of the build, plus Hq >= 1, Hq % Hkv == 0,
 * G = Hq / Hkv <= 16, 1 <= T <= L and a finite sm_scale.
 *
 * Every decode entry point enqueues two launches on `stream`: the query hash
 * (which also resets the decode's counters in the workspace), then one launch
 * that counts collisions, selects, attends and merges.  Workgroups of that
 * launch hand results to each other through the workspace and wait for each
 * other with bounded polls; a wait that does not end (which correct use never
 * causes) writes NaN into the affected outputs instead of hanging.  The
 * workspace must not be used by another call that may run at the same time.
 * The probe reads `indices` in aligned 16-byte blocks, so it may read up to
 * 14 bytes before the first or after the last entry of a probed bucket (never
 * outside the 16-byte-aligned block holding an entry of the array); those
 * bytes are never used.
 * ---------------------------------------------------------------------- */

/* Bytes of device workspace lsh_decode_attention needs (0 on invalid sizes).
 * The size never decreases with N, so the size at a cache's capacity serves
 * every decode over a shorter prefix of it. */
size_t lsh_decode_workspace_size(int B, int Hq, int Hkv, int N, int d, int K,
                                 int L, int stride);

/*
 * q        [B, Hq, d]      dtype        one decode query per head
 * keys, values [B, Hkv, N, d] dtype     the cache the tables were built from
 * W        [d, L*K]        dtype        the build's projection
 * indices, offsets                      the build's outputs (built with the same
 *                                       stride)
 * out      [B, Hq, d]      float        out: the estimate
 * lse      [B, Hq]         float        optional out: natural-log log-sum-exp
 * nsel     [B, Hq]         int32        optional out: |S|
 * q_codes  [B, Hq, L]      uint16       optional out: code_l(q)
 * counts   [B, Hq, N]      uint8        optional out: collision counts c(n)
 */
lsh_status lsh_decode_attention(const void* q, const void* keys,
                                const void* values, const void* W,
                                const uint16_t* indices, const uint16_t* offsets,
                                int B, int Hq, int Hkv, int N, int d, int K,
                                int L, int T, int stride, float sm_scale,
                                int dtype,
                                float* out, float* lse, int32_t* nsel,
                                uint16_t* q_codes, uint8_t* counts,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Hybrid decode: exact attention over a static set of keys, the LSH estimate
 * over the rest.  MagicPIG pairs dense attention with sampled sparse
 * attention ("How infini-ai-lab/magicpig works", overview; sourcepulse
 * summary, "How It Works"); the static set taken here is the first n_sink
 * keys (attention sinks) and the last n_window keys (the recent window), the
 * keys MAC-Attention recomputes exactly and merges by log-sum-exp
 * ("MAC-Attention" README, "How It Works").
 *
 *   E    = { n : n < n_sink } U { n : n >= N - n_window }
 *   S'   = S \ E                (selected keys outside the exact set)
 *   out  = sum_{n in E} e^{s q.k_n} v_n + sum_{n in S'} e^{l(n)} v_n,
 *          divided by the same sum without v_n;  lse = ln of that sum
 *          (l(n) as in lsh_decode_attention; E and S' empty: out = 0,
 *          lse = -inf)
 *   nsel = |S'|;  counts (optional) are the collision counts of every key.
 *
 * Arguments are those of lsh_decode_attention plus n_sink, n_window >= 0
 * (LSH_ERR_INVALID_ARG if negative; values past N are clamped).  The exact
 * set is attended in at most 16 pieces, one workgroup per piece and
 * (sequence, kv head), for all query heads of the group at once: it reads
 * each of its keys and values once per kv head.  n_sink = n_window = 0 is
 * lsh_decode_attention.  Same workspace size.
 */
lsh_status lsh_decode_attention_hybrid(const void* q, const void* keys,
                                       const void* values, const void* W,
                                       const uint16_t* indices, const uint16_t* offsets,
                                       int B, int Hq, int Hkv, int N, int d, int K,
                                       int L, int T, int stride, float sm_scale,
                                       int dtype, int n_sink, int n_window,
                                       float* out, float* lse, int32_t* nsel,
                                       uint16_t* q_codes, uint8_t* counts,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * Decode over a cache with room for n_cap keys: the hybrid decode above, for
 * sequence b over its first len_b keys, with keys, values [B, Hkv, n_cap, d]
 * and tables of the pitch lsh_update_tables uses (indices [B, Hkv, L, n_cap],
 * offsets [B, Hkv, L, lsh_num_chunks(n_cap, stride), 2^K]) holding exactly
 * those keys (built or updated to len_b).
 *
 * seq_lens [B] int32   optional (device): len_b, clamped into [0, N]; NULL:
 *                      every len_b = N.  N is the longest; the launch covers N.
 * w_per_head           W as in lsh_update_tables (0 shared, 1 per kv head).
 * counts               when given, [B, Hq, N]; 0 for keys at or past len_b.
 *
 * Keys and values of sequence b from position len_b on are never read.  The
 * exact set of sequence b is its first min(n_sink, len_b) keys and the last
 * n_window of the rest (E of the hybrid decode with N = len_b); a sequence
 * with len_b = 0 gets out = 0, lse = -inf, nsel = 0.  N <= n_cap and
 * w_per_head in {0, 1}, else LSH_ERR_INVALID_ARG.  Workspace:
 * lsh_decode_workspace_size at N (or at n_cap, which is never smaller).
 * lsh_decode_attention_hybrid is this call with n_cap = N, no lengths and a
 * shared W.
 */
lsh_status lsh_decode_attention_cached(const void* q, const void* keys,
                                       const void* values, const void* W,
                                       const uint16_t* indices, const uint16_t* offsets,
                                       int B, int Hq, int Hkv, int N, int n_cap,
                                       const int32_t* seq_lens,
                                       int d, int K, int L, int T, int stride,
                                       float sm_scale, int dtype, int w_per_head,
                                       int n_sink, int n_window,
                                       float* out, float* lse, int32_t* nsel,
                                       uint16_t* q_codes, uint8_t* counts,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * The cached decode above with no workspace argument and no allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Arguments and
 * results are those of lsh_decode_attention_cached without workspace and
 * workspace_bytes.
 *
 * The workspace is a static device array of LSH_NOALLOC_SCRATCH_BYTES (64 MiB)
 * inside the library, one per device the library runs on, held until the
 * process ends; its device address is looked up once per device, on the
 * first call made with that device current.  A call that needs more
 * (lsh_decode_workspace_size above the limit) returns LSH_ERR_WORKSPACE and
 * launches nothing.  The call allocates nothing: no hipMalloc, no hipFree, no
 * host allocation.  Its launches are never timed by the kernel-timing window
 * below (taking events for them could allocate).
 *
 * Every call on a device shares that device's array, which keeps the last
 * call's contents (the decode clears what must start at zero itself): calls
 * that may overlap on one device (other streams, other threads) race, and
 * must be ordered by the caller.
 */
#define LSH_NOALLOC_SCRATCH_BYTES (64u << 20)
lsh_status lsh_decode_attention_noalloc(const void* q, const void* keys,
                                        const void* values, const void* W,
                                        const uint16_t* indices, const uint16_t* offsets,
                                        int B, int Hq, int Hkv, int N, int n_cap,
                                        const int32_t* seq_lens,
                                        int d, int K, int L, int T, int stride,
                                        float sm_scale, int dtype, int w_per_head,
                                        int n_sink, int n_window,
                                        float* out, float* lse, int32_t* nsel,
                                        uint16_t* q_codes, uint8_t* counts,
                                        void* stream);

/* ------------------------------------------------------------------------
 * Launch printing (a debugging aid): with the environment variable
 * LSH_DEBUG_LAUNCH set to anything but "" or "0" when the library first
 * launches, every launch prints one line to stderr with the kernel's name,
 * grid, block, dynamic LDS bytes and stream.
 * ---------------------------------------------------------------------- */

/* ------------------------------------------------------------------------
 * Kernel timing (a profiling aid; process-wide, one window at a time)
 *
 * Between lsh_timing_begin() and lsh_timing_end() every kernel the library
 * launches carries a start and a stop event on its own dispatch, so the
 * measured time is the kernel's execution on the GPU, with no extra work on
 * the stream.  Events come from a host-side pool that grows on demand and is
 * kept for reuse (no device memory).
 * ---------------------------------------------------------------------- */

/* Number of kernel kinds; ids run 0 .. lsh_kernel_count() - 1. */
int lsh_kernel_count(void);

/* Name of kernel kind `id` (static string), or NULL for an invalid id. */
const char* lsh_kernel_name(int id);

/* Opens a timing window.  LSH_ERR_INVALID_ARG if one is already open. */
lsh_status lsh_timing_begin(void);

/* Closes the window: waits for every timed launch and writes, per kernel
 * kind, the summed execution time in milliseconds and the number of
 * launches into HOST arrays of lsh_kernel_count() entries (either may be
 * NULL).  LSH_ERR_INVALID_ARG if no window is open, LSH_ERR_HIP if an event
 * could not be read (those launches are left out of the sums). */
lsh_status lsh_timing_end(double* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* LSH_ATTN_H */
