/*
 * loopkv.h -- C ABI of the LoopKV plan-driven quantized decode library for
 * MI355X (gfx950).
 *
 * What the library computes comes from "LoopKV: Loop-Aware KV Cache
 * Compression for Serving Looped Transformers", abstract (概要):
 *   - every (loop, layer) cell of a looped transformer has its own KV cache;
 *   - a plan fixed ahead of time keeps a cell at 4 bits or at 2 bits, or
 *     lets it borrow the last loop's cache of the same layer;
 *   - a decoding loop always uses the upper two bits of a 4-bit value and
 *     loads the lower two only for tokens whose weight under that loop's own
 *     query is large enough to need them.
 * The quantizer layout (keys per channel over token groups, values per token
 * over channel groups, fp16 scale and zero point) follows the KIVI entry of
 * the related-papers list on the fugumt LoopVQ page.
 *
 * Conventions for every call
 *   - All pointers documented "device" are HIP device pointers owned by the
 *     caller; "host" pointers are read during the call only.  The library
 *     never allocates or frees device memory.  It owns the host-side,
 *     immutable plan object and one fixed device array per GPU, the scratch
 *     of loopkv_decode_noalloc (part of its loaded code object).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Compute calls are asynchronous on that stream: launch errors are
 *     reported by the return code, faults surface at the caller's next
 *     synchronization.
 *   - Return codes: 0 = LOOPKV_OK, > 0 = informational success,
 *     < 0 = error with nothing launched.  loopkv_last_error() returns the
 *     calling thread's last error message.  No call aborts or throws.
 *   - Host-visible arguments are always validated.  Device-resident lengths
 *     and block tables are trusted (an out-of-range entry is undefined
 *     behaviour) unless the environment variable LOOPKV_DEBUG=1 is set, in
 *     which case they are copied to the host and checked first (this
 *     synchronizes the stream; an out-of-range entry then fails the call
 *     with LOOPKV_E_INVAL before any launch).  LOOPKV_LOG=1 prints one line
 *     per append / decode call to stderr: the cell, its source and mode,
 *     the split layout and the plan-required bytes of the split pass (from
 *     sum_seq_lens when given, else for max_seq_len per sequence).  Both
 *     variables are read on every call.
 *   - The plan is immutable: concurrent calls on different streams are safe
 *     when they write different pools / workspaces.
 *
 * Data layout (all little-endian)
 *   G = 32 (key-group tokens and value-group channels), P = page tokens,
 *   D = head_dim, row = D/4 bytes (2-bit codes, channel 4k+i in bits
 *   [2i,2i+1] of byte k).
 *   Pool of one stored cell: H x num_pages head-blocks, head-major: head h
 *   of physical page p starts at byte (h*num_pages + p) * HB.
 *   4-bit head-block: K_hi[P rows] K_lo[P rows] V_hi[P rows] V_lo[P rows]
 *                     Vmeta[P][D/G]{fp16 scale, fp16 zero}
 *                     Kmeta[max(1,P/G) slots]{fp16 scale[D], fp16 zero[D]}
 *   2-bit head-block: K[P rows] V[P rows] Vmeta Kmeta.
 *   Key group g (tokens 32g..32g+31) keeps its metadata in the page holding
 *   token 32g, slot (32g mod P)/32.  A 4-bit code c is stored as
 *   hi = c >> 2 in the *_hi plane and lo = c & 3 in the *_lo plane.
 */
#ifndef LOOPKV_H
#define LOOPKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOOPKV_ABI_VERSION 1

enum {
  LOOPKV_OK = 0,
  LOOPKV_NOOP_REUSE = 1,   /* append on a reuse cell: nothing to store     */
  LOOPKV_E_INVAL = -1,     /* bad argument                                  */
  LOOPKV_E_PLAN = -2,      /* malformed or invalid plan blob                */
  LOOPKV_E_CAPACITY = -3,  /* workspace / staging / pool too small          */
  LOOPKV_E_HIP = -4        /* HIP runtime error (message has HIP's text)    */
};

enum { LOOPKV_CELL_Q4 = 0, LOOPKV_CELL_Q2 = 1, LOOPKV_CELL_REUSE = 2 };

typedef struct loopkv_plan loopkv_plan; /* opaque, host, immutable */

/* ABI version compiled into the library (compare with LOOPKV_ABI_VERSION). */
int loopkv_abi_version(void);

/* Thread-local text of the last error ("" if none).  Valid until the next
 * call on the same thread. */
const char* loopkv_last_error(void);

/*
 * loopkv_plan_load -- parse the per-cell plan.
 * Source: LoopKV abstract -- the offline profile picks 4-bit, 2-bit or
 * final-loop reuse for every (loop, layer) cell; a threshold tau per cell
 * decides where the low bits are fetched.
 * blob (host, nbytes): "LKVP", u32 version = 1, i32 R, L, H, D, G, P, then
 *   R*L records {u8 kind, u8 pad[3], f32 tau} in [loop][layer] order.
 * Accepted: 1 <= R, L <= 4096, 1 <= H <= 1024, D in {64, 128}, G == 32,
 *   P in {16, 32, 64}; kind in {Q4, Q2, REUSE}; REUSE only in loops
 *   0..R-2; tau >= 0 or +inf, never NaN.
 * out: receives a new plan (free with loopkv_plan_free).
 * Errors: LOOPKV_E_INVAL for NULL pointers, LOOPKV_E_PLAN otherwise.
 */
int loopkv_plan_load(const void* blob, size_t nbytes, loopkv_plan** out);
void loopkv_plan_free(loopkv_plan* plan);

/* dims[6] <- R, L, H, D, G, P.  Errors: LOOPKV_E_INVAL. */
int loopkv_plan_dims(const loopkv_plan* plan, int32_t dims[6]);

/* Cell (loop, layer): its kind, its tau and the loop of the cell whose
 * cache it reads (R-1 for REUSE, else `loop`).  Any output may be NULL. */
int loopkv_cell_info(const loopkv_plan* plan, int loop, int layer,
                     int* kind, float* tau, int* src_loop);

/* Bytes of one head-block (HB) of the cell's pool; 0 for REUSE or bad args. */
size_t loopkv_head_block_bytes(const loopkv_plan* plan, int loop, int layer);

/* Bytes of a pool of num_pages pages (H * num_pages * HB); 0 for REUSE. */
size_t loopkv_pool_bytes(const loopkv_plan* plan, int loop, int layer,
                         int64_t num_pages);

/* Bytes of the key staging buffer of a stored cell for max_slots
 * sequences: max_slots * H * 32 * D bf16 (raw keys of each sequence's open,
 * incomplete key group).  0 for REUSE. */
size_t loopkv_staging_bytes(const loopkv_plan* plan, int loop, int layer,
                            int32_t max_slots);

/* Device workspace bytes loopkv_decode needs for `batch` sequences of at
 * most max_seq_len tokens (any cell of the plan, any split count).  No
 * initial contents are needed.  Calls sharing one workspace must not run
 * concurrently (stream-order them). */
size_t loopkv_decode_workspace_bytes(const loopkv_plan* plan, int32_t batch,
                                     int32_t max_seq_len);

/* The split layout loopkv_decode uses for a batch with these host fields
 * (batch, max_seq_len, sum_seq_lens as in loopkv_batch) and num_splits
 * (0 = automatic), for a cell with a tau mask or none: out[0] = partial
 * records per (sequence, head) (the splits of a uniform layout), out[1] =
 * tokens per split (per wave range of a streamed layout; see
 * loopkv_decode_layout).  Every layout has out[1] a multiple of 64,
 * out[1] <= 4096, out[1] <= max_seq_len rounded up to 64, out[0] <= 2048
 * and out[0] * out[1] >= max_seq_len; the workspace size above holds the
 * partial records and candidate lists of any such layout.  The automatic
 * choice depends on the current device's compute-unit count (256 when no
 * device is visible).  Errors: LOOPKV_E_INVAL (NULL argument, negative
 * sizes, or a num_splits / max_seq_len that needs more than 2048 splits). */
int loopkv_decode_splits(const loopkv_plan* plan, int32_t batch, int32_t max_seq_len,
                         int32_t sum_seq_lens, int32_t num_splits, int32_t out[2]);

/* The split layout loopkv_decode uses for cell (loop, layer) and these host
 * fields: out[0] = 0 for a uniform layout (every (sequence, head) cut into
 * out[1] splits of out[2] tokens, as loopkv_decode_splits reports) or 1 for
 * a streamed one: the pairs' 64-token tiles laid end to end (sequence-major,
 * then head) and cut into ranges, the first ranges (about 90% of the tiles
 * by the length-sum hint, one per resident wave slot) of out[2] / 64 tiles,
 * the rest of 16; out[3] waves take one range each, and ranges past the
 * grid (a hint below the real sum leaves some) go to the last wave in turn.
 * A pair gets one partial record per range that meets it, at most out[1].
 * Streamed layouts serve ragged batches (a length sum below 85% of
 * batch * max_seq_len) of at most 256 sequences with a tau mask or none
 * (not tau = 0).  Errors: LOOPKV_E_INVAL as loopkv_decode_splits, or a bad
 * cell. */
int loopkv_decode_layout(const loopkv_plan* plan, int loop, int layer, int32_t batch, int32_t max_seq_len,
                         int32_t sum_seq_lens, int32_t num_splits, int32_t out[4]);

/* Memory of one cell; an array of R*L of these is indexed [loop*L + layer].
 * REUSE cells may leave everything NULL / 0. */
/* Limit: one head's region of a pool, num_pages * head-block bytes, must
 * stay below 4 GiB (decode addresses it with 32-bit offsets). */
typedef struct {
  void* pool;          /* device, loopkv_pool_bytes(num_pages) bytes         */
  void* staging;       /* device, loopkv_staging_bytes(max_slots) bytes      */
  int64_t num_pages;   /* pages in this pool (shared page numbering)         */
  int32_t max_slots;   /* staging slots                                      */
  int32_t reserved;
} loopkv_cell_mem;

/* One batch of sequences.  Every cell uses the same page mapping.  The
 * device arrays are int32 and must be 4-byte aligned; every call rejects a
 * batch above 65535 sequences (LOOPKV_E_INVAL). */
typedef struct {
  int32_t batch;                /* number of sequences, 0 <= B <= 65535      */
  int32_t max_pages;            /* row stride of block_tables                */
  const int32_t* seq_lens;      /* device [B]: append = length BEFORE the
                                   append; decode = tokens attended          */
  const int32_t* slots;         /* device [B] staging slot per sequence, or
                                   NULL for slot = sequence index            */
  const int32_t* block_tables;  /* device [B][max_pages]: logical page ->
                                   physical page (0 <= p < num_pages)        */
  int32_t max_seq_len;          /* host upper bound of the lengths involved
                                   (decode: attended; append: after append)  */
  int32_t sum_seq_lens;         /* optional host hint: sum of the attended
                                   lengths (0 = unknown).  Decode uses it only
                                   to size splits for ragged batches; any
                                   value gives correct results.              */
} loopkv_batch;

/*
 * loopkv_append -- quantize and store n_new new tokens of every sequence in
 * cell (loop, layer).
 * Source: LoopKV abstract (cells stored at 4 or 2 bits; 4-bit values kept
 * as separately readable high and low bit planes).
 * k_bf16, v_bf16: device [B][n_new][H][D] bfloat16 (raw keys and values of
 *   tokens seq_lens[b] .. seq_lens[b]+n_new-1), 16-byte aligned.
 * Effects: value rows and metadata of the new tokens; key codes and key
 *   metadata of every key group the new tokens touch (the open group of a
 *   sequence is re-quantized over all its tokens, read back from staging);
 *   staging then holds the raw keys of each sequence's open group.
 *   Pages for all tokens < seq_lens[b] + n_new must be mapped.  Values must
 *   be finite with |x| <= 32768.
 * Returns LOOPKV_NOOP_REUSE (nothing launched) for a reuse cell.
 * Errors: LOOPKV_E_INVAL (bad cell, NULL pool/staging, n_new < 1,
 *   misaligned inputs or batch arrays, batch above 65535,
 *   max_pages * P < max_seq_len), LOOPKV_E_CAPACITY (batch > max_slots
 *   when slots == NULL), LOOPKV_E_HIP.
 */
int loopkv_append(const loopkv_plan* plan, const loopkv_cell_mem* cells,
                  int loop, int layer, const loopkv_batch* batch,
                  int32_t n_new, const void* k_bf16, const void* v_bf16,
                  void* stream);

typedef struct {
  float sm_scale;              /* score = sm_scale * q . k                    */
  int32_t num_splits;          /* splits per (sequence, head); 0 = automatic  */
  void* workspace;             /* device, loopkv_decode_workspace_bytes       */
  size_t workspace_bytes;
  uint32_t* mask_bits;         /* optional device [B][H][ceil(max_seq_len/32)]:
                                  bit t of a (b, h) row = low plane of token t
                                  fetched (all ones up to T for tau = 0)      */
  unsigned long long* counters;/* optional device [2], accumulated with
                                  atomics: [0] flagged token-heads,
                                  [1] low-plane bytes read                    */
} loopkv_decode_opts;

/*
 * loopkv_decode -- one decode step of cell (loop, layer) for every sequence.
 * Source: LoopKV abstract -- the cell reads its source cache (itself, or
 * the final loop's cell of its layer for REUSE), dequantizes keys at the
 * source's precision, forms softmax weights from its own query, reads the
 * high plane of every value and fetches the low plane only of tokens whose
 * own weight p_t >= tau of the calling cell.  An unfetched 4-bit value is
 * reconstructed at its bucket centre (4*hi + 3/2)*s + z.
 * q_bf16: device [B][H][D] bfloat16.  out: device [B][H][D] float32.
 * A sequence of length 0 produces zeros.  A (sequence, head) is cut into
 * at most 2048 splits of at most 4096 tokens, so max_seq_len is limited to
 * 8,388,608.
 * Alignment: q 2 bytes, out and mask_bits 4 bytes, counters 8 bytes.
 * Errors: LOOPKV_E_INVAL (bad cell, NULL pointers, misaligned pointers,
 *   batch above 65535, num_splits < 0, sm_scale not finite,
 *   max_pages * P < max_seq_len, more than 2048 splits, which a
 *   max_seq_len above the limit or a large num_splits asks for),
 *   LOOPKV_E_CAPACITY (workspace too small), LOOPKV_E_HIP.
 */
int loopkv_decode(const loopkv_plan* plan, const loopkv_cell_mem* cells,
                  int loop, int layer, const loopkv_batch* batch,
                  const void* q_bf16, float* out,
                  const loopkv_decode_opts* opts, void* stream);

/*
 * loopkv_decode_noalloc -- loopkv_decode for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results as
 * loopkv_decode (bit for bit), except that opts->workspace and
 * opts->workspace_bytes are ignored: the split partials, candidate counts
 * and candidate lists live in a device array the library holds, one copy of
 * LOOPKV_NOALLOC_SCRATCH_BYTES per GPU it runs on, until the process ends.
 * The call allocates nothing.  loopkv_decode_noalloc_bytes gives the bytes
 * a call with these host fields would use (0 for invalid arguments); a
 * batch that needs more fails with LOOPKV_E_CAPACITY before any launch.
 * No initial contents are needed.  Every call on one GPU uses that GPU's
 * copy: calls that overlap on one GPU (on different streams, or from host
 * threads without stream ordering) race and give undefined results.
 * Errors: as loopkv_decode; LOOPKV_E_CAPACITY when the batch needs more
 *   than LOOPKV_NOALLOC_SCRATCH_BYTES.
 */
#define LOOPKV_NOALLOC_SCRATCH_BYTES (32u << 20)
size_t loopkv_decode_noalloc_bytes(const loopkv_plan* plan, int loop, int layer, int32_t batch,
                                   int32_t max_seq_len, int32_t sum_seq_lens, int32_t num_splits);
int loopkv_decode_noalloc(const loopkv_plan* plan, const loopkv_cell_mem* cells,
                          int loop, int layer, const loopkv_batch* batch,
                          const void* q_bf16, float* out,
                          const loopkv_decode_opts* opts, void* stream);

/*
 * loopkv_plan_optimize -- offline plan search: the kind of every cell that
 * minimizes decode reads under a damage budget and a storage budget.
 * Source: LoopKV abstract -- the model's output damage is close to the sum
 * of per-cell damages; per cell a profile taken once, offline, selects
 * 4-bit codes, 2-bit codes or borrowing the last loop's cache, and the plan
 * reads the fewest bytes within limits on predicted damage and storage.
 * damage: host [R][L][4] doubles per cell (loop-major): predicted damage
 *   when the cell is stored at 4 bits, at 2 bits, when it reuses a 4-bit
 *   final-loop cell, when it reuses a 2-bit one (the reuse entries of loop
 *   R-1 are ignored).  Finite, >= 0.
 * Costs per token-head in 32-byte units (head_dim 128): reads 4 (a 4-bit
 *   source: both key planes, high value plane, metadata) or 3 (2-bit);
 *   a reuse cell reads its source's format.  Storage 5 (4-bit: four planes
 *   + metadata), 3 (2-bit), 0 (reuse).  Low-plane fetches of flagged tokens
 *   are not counted.
 * Result: among plans with total damage <= damage_budget and total storage
 *   <= storage_budget, the one with least reads, then least damage, then
 *   least storage.  kinds: host out [R][L] LOOPKV_CELL_* (reuse never in
 *   loop R-1).  totals: host out [3] (reads, storage, damage), may be NULL.
 * The search is exact (dynamic program over layers; O(L * (20R L)^2 / 3)
 *   time for R = 4).
 * Errors: LOOPKV_E_INVAL (R not in 1..8, L not in 1..4096, NULL pointers,
 *   negative / non-finite inputs, instance too large, host memory for the
 *   search tables not available), LOOPKV_E_PLAN (no
 *   plan meets both budgets).
 */
int loopkv_plan_optimize(int32_t R, int32_t L, const double* damage, double damage_budget,
                         int64_t storage_budget, uint8_t* kinds, double* totals);

/*
 * ---- Joint vector quantization across loop steps (LoopVQ-style) ---------
 * Source: "LoopVQ: Sub 1-bit KV Cache Quantization for Looped
 * Transformers", abstract -- keys and values change little from one loop
 * step to the next, so one codebook entry stands for a group of channels
 * of all loop steps at once, at half a bit per element.
 * Format of one layer (all R loops share it): for a token and head, channel
 * group j (channels 4j..4j+3, j < D/4) has a joint vector of 4R numbers,
 * loop r's channels at positions 4r..4r+3; its key (value) index is one
 * byte naming the nearest of 256 codewords of group j's key (value)
 * codebook.  R = 4 gives 8 bits per 16 elements = 0.5 bit per element.
 * Codebook (one layer, keys or values): device fp16 [R][256][D/4][4], loop
 *   r's 4 channels of codeword c of group j at ((r*256 + c)*(D/4) + j)*4,
 *   so one loop's slices of all codewords are one contiguous block.  The
 *   joint codeword c of group j is the concatenation over r = 0 .. R-1.
 * Pool: device, head-major like the cell pools: head h of physical page p
 *   at byte (h*num_pages + p) * 2*P*(D/4); inside, P key index rows of D/4
 *   bytes (token-major), then P value index rows of D/4 bytes.  A row is
 *   XOR-rotated by the token's position: group j of the token at sequence
 *   position t (in-page slot t mod P) is byte j ^ (t mod (D/4)) of its row
 *   (key at (t mod P)*(D/4) + (j ^ (t mod D/4)), value P*(D/4) further).
 */
typedef struct {
  int32_t loops;       /* R, 2..4 */
  int32_t heads;       /* H, 1..1024 (the decode grid carries heads in a
                          dimension of at most 65535 blocks; 1024 as for plans) */
  int32_t head_dim;    /* D, 64 or 128 */
  int32_t page;        /* P, 16, 32 or 64 */
} loopkv_vq_dims;

/* Bytes of one codebook, of a pool of num_pages pages, and of the decode
 * workspace (no initial contents needed); 0 for invalid dims. */
size_t loopkv_vq_codebook_bytes(const loopkv_vq_dims* dims);
size_t loopkv_vq_pool_bytes(const loopkv_vq_dims* dims, int64_t num_pages);
size_t loopkv_vq_workspace_bytes(const loopkv_vq_dims* dims, int32_t batch, int32_t max_seq_len);

/*
 * loopkv_vq_append -- code n_new new tokens of every sequence: each joint
 * vector gets the index of its nearest codeword (squared Euclidean distance
 * in fp32, ties to the lowest index).
 * k_bf16, v_bf16: device [R][B][n_new][H][D] bfloat16, all loops' keys and
 *   values of tokens seq_lens[b] .. seq_lens[b]+n_new-1, 8-byte aligned.
 * codebook_k / codebook_v: device fp16 [R][256][D/4][4], 8-byte aligned.
 * Pages for all tokens < seq_lens[b] + n_new must be mapped.
 * Errors: LOOPKV_E_INVAL (bad dims, NULL pointers, n_new < 1, misaligned
 *   inputs or batch arrays, batch above 65535, max_pages * P <
 *   max_seq_len), LOOPKV_E_HIP.
 */
int loopkv_vq_append(const loopkv_vq_dims* dims, void* pool, int64_t num_pages,
                     const void* codebook_k, const void* codebook_v,
                     const loopkv_batch* batch, int32_t n_new,
                     const void* k_bf16, const void* v_bf16, void* stream);

/*
 * loopkv_vq_decode -- one decode step of loop `loop` over a layer's joint
 * cache: keys and values are the loop's slices (positions 4*loop ..
 * 4*loop+3) of the chosen codewords; o = softmax(sm_scale * q.K^) V^.
 * q_bf16: device [B][H][D] bfloat16 (8-byte aligned); codebooks as for
 * loopkv_vq_append but 16-byte aligned; out: device fp32 [B][H][D].  A
 * sequence of length 0 produces zeros.  The summation
 * order is fixed by the launch shape, so repeated calls with the same
 * inputs and workspace size give identical bits.
 * Errors: LOOPKV_E_INVAL (bad dims or loop, NULL or misaligned pointers,
 *   batch above 65535, sm_scale not finite, max_pages * P < max_seq_len),
 *   LOOPKV_E_CAPACITY (workspace too small), LOOPKV_E_HIP.
 */
int loopkv_vq_decode(const loopkv_vq_dims* dims, const void* pool, int64_t num_pages,
                     const void* codebook_k, const void* codebook_v, int loop,
                     const loopkv_batch* batch, const void* q_bf16, float* out,
                     float sm_scale, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Measurement hook (not an operation of the method; used by benchmarks to
 * time kernels live).  While enabled, every kernel launch this library makes
 * carries a pair of HIP events that the runtime stamps with that kernel's
 * own start and end on the launch's stream (hipExtLaunchKernel); nothing is
 * recorded between launches, so kernels run back to back as they do
 * unprofiled.  An append's interval runs from its first kernel's start to
 * its last kernel's end.
 * loopkv_profile_collect waits for the recorded events of one kernel class
 * (LOOPKV_KERNEL_*), returns the number of launches and their summed
 * duration in milliseconds, and clears that class.  Enabling/disabling is
 * process-wide; the events are created by the library on first use and
 * reused.  Errors: LOOPKV_E_INVAL (bad class or NULL output), LOOPKV_E_HIP.
 */
enum { LOOPKV_KERNEL_SPLIT = 0, LOOPKV_KERNEL_MERGE = 1, LOOPKV_KERNEL_APPEND = 2 };
int loopkv_profile_enable(int on);
int loopkv_profile_collect(int kernel_class, int64_t* launches, double* total_ms);

/*
 * Measurement helper (not an operation of the method): reads `bytes` (a
 * multiple of 16, rounded down) from device buffer `buf` with 16-byte loads
 * on `stream`, to measure the practical HBM read bandwidth next to the
 * nominal peak.  `sink` (device, may be NULL) is written only for one
 * impossible checksum, so the loads cannot be optimized away.
 * Errors: LOOPKV_E_INVAL (NULL or unaligned buffer), LOOPKV_E_HIP.
 */
int loopkv_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LOOPKV_H */
