/*
 * sink_attn.h -- C ABI of libsinkattn.so: attention whose softmax
 * denominator carries one extra "sink" logit per query head, forward and
 * backward, over packed variable-length (THD) sequences, for AMD MI355X
 * (gfx950).
 *
 * What is computed. For each sequence b, q-head h (kv-head hk = h / (Hq/Hk))
 * and query row i, with S_ij = scale * q_i . k_j over the kept keys j:
 *
 *   out_i = sum_j e^{S_ij} v_j / (e^{s_h} + sum_j e^{S_ij})
 *   lse_i = ln(e^{s_h} + sum_j e^{S_ij})              (sink INCLUSIVE)
 *
 * i.e. softmax over the scores with the sink s_h appended as one more
 * column, that column dropped afterwards ("slime: learnable_softmax_
 * attention.py", module docstring), evaluated in the max-stabilised form
 * m = max(s_h, max_j S_ij) of the "CANN ops-transformer: flash_attn" page
 * (Formula section). softmax_n ("Flash-Attention-Softmax-N" README,
 * introduction) is the special case s_h = ln n; s_h = -inf (or a NULL sink
 * pointer) is plain softmax attention. The sink is not multiplied by scale.
 *
 * Masks ("pytorch/pytorch issue #108108", Proposal section): row i stands
 * at key position p_i = i + (Lk_b - Lq_b) (bottom-right alignment).
 * causal keeps j <= p_i; win_right >= 0 keeps j <= p_i + win_right;
 * win_left >= 0 keeps j >= p_i - win_left (inclusive; -1 = unbounded, as in
 * the "slime" wrapper's window_size and the CANN page's win_left/win_right).
 * causal requires win_right in {-1, 0}. A row that keeps no key gets
 * out = 0 and lse = s_h (-inf without a sink; its gradients are then 0).
 *
 * Backward ("slime", _LearnableSoftmaxFlashAttnVarlen.backward, and the
 * chain rule through the extended softmax): with P_ij = e^{S_ij - lse_i},
 * D_i = dO_i . out_i and dS_ij = P_ij (dO_i . v_j - D_i):
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
 *   dv_j = sum_i P_ij dO_i  (dk, dv summed over the q-heads of a group),
 *   dsink_h = -sum_i e^{s_h - lse_i} D_i.
 * D_i is formed from the stored out (in the input dtype), as the "slime"
 * page's backward feeds its rounded output to the vanilla backward. For a
 * single head, dsink is a sum of random-sign terms over all of that head's
 * rows and can cancel by two orders of magnitude; the rounding of out to
 * bf16 (at most half a bf16 step per element) then moves it by a few
 * percent of its value (about 5% on one head of a 32k-token causal batch),
 * while the [num_heads_q] vector as a whole stays within 2e-2 relative L2 of
 * the exact gradient. In fp32, dsink is exact to about 1e-5 of the sum of
 * its terms' magnitudes.
 * Windows of max_seqlen_q + max_seqlen_k or more exclude no key and are
 * treated as unbounded.
 *
 * Layouts (all contiguous, row-major, base pointers 16-byte aligned). The
 * packed TND layout of the sink_attn_fwd / _bwd / _fwd_paged calls:
 *   q, out, dout, dq : [total_q, num_heads_q, head_dim]  (dtype)
 *   k, v, dk, dv     : [total_k, num_heads_k, head_dim]  (dtype)
 *   lse              : [num_heads_q, total_q] fp32
 *   sink_logits, dsink: [num_heads_q] fp32
 *   cu_seqlens_q/k   : [batch + 1] int32, first 0, non-decreasing,
 *                      last = total ("slime" wrapper docstring; CANN page,
 *                      SeqLengths parameter group)
 * and the batch-padded layouts of the *_padded calls (CANN page, q, k, v
 * validation and the layout matching table), with S_q = seq_q, S_k = seq_k:
 *   BSND: q, dq [batch, S_q, num_heads_q, head_dim]; k, v, dk, dv
 *         [batch, S_k, num_heads_k, head_dim]
 *   BNSD: q, dq [batch, num_heads_q, S_q, head_dim]; k, v, dk, dv
 *         [batch, num_heads_k, S_k, head_dim]
 *   out, dout: layout_out (BSND or BNSD) of q's shape
 *   lse  : [batch, num_heads_q, S_q] fp32
 *   seqused_q / seqused_kv: [batch] int32, rows of sequence b in use
 *         (0 <= used <= S; NULL: all S). Rows past them are padding: they
 *         are never read, and out, lse, dq, dk, dv keep whatever they held
 *         there.
 *
 * Ownership and threading. The library allocates nothing and keeps no state
 * between calls (except the one-shot timing events of sink_attn_arm_timing,
 * which are per host thread). Every device buffer and the stream belong to
 * the caller; fwd/bwd only enqueue work on `stream` and return, so device
 * buffers, meta_dev and workspace must stay alive until that work is done.
 * Outputs must not alias inputs. Calls are reentrant.
 *
 * Errors. Every argument the host can see is checked and reported through
 * the returned status; nothing is thrown across the ABI and nothing is
 * launched when a check fails. Values that live only in device memory
 * (device cu_seqlens equal to the host copy used for the metadata, NaN
 * inputs) are not checked: passing inconsistent ones is undefined, as on
 * the CANN page (Constraints, "Declaration").
 */
#ifndef SINK_ATTN_H
#define SINK_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SINK_ATTN_ABI_VERSION 5

/* Index of the metadata header word that holds the length (in words) of the
 * table prefix the forward calls read. */
#define SINK_ATTN_META_FWD_WORDS 47

typedef enum {
  SINK_ATTN_OK = 0,
  SINK_ATTN_E_INVALID = 1,          /* bad argument value or pointer        */
  SINK_ATTN_E_UNSUPPORTED = 2,      /* head_dim or dtype not built          */
  SINK_ATTN_E_META_MISMATCH = 3,    /* metadata header differs from call    */
  SINK_ATTN_E_BUFFER_TOO_SMALL = 4, /* meta capacity or workspace too small */
  SINK_ATTN_E_HIP = 5               /* a HIP launch failed                  */
} sink_attn_status;

/* Element type of q, k, v, out, dout, dq, dk, dv (lse, sinks, dsink are
 * always fp32). fp16 is the CANN page's other input type (q, k, v
 * validation); it runs the same MFMA kernels as bf16. fp32 runs a plain
 * VALU path, one thread per query row (or key row in the dK/dV pass), with
 * no tile schedule and no MFMA: it serves as the exact-arithmetic
 * configuration for small problems and is orders of magnitude slower than
 * the 16-bit path on long sequences. */
typedef enum { SINK_ATTN_FP32 = 0, SINK_ATTN_BF16 = 1, SINK_ATTN_FP16 = 2 } sink_attn_dtype;

/* Tensor layouts (CANN page, layout matching table): k and v always share
 * q's layout; out may differ from q only as BNSD q with BSND out. */
typedef enum { SINK_ATTN_TND = 0, SINK_ATTN_BSND = 1, SINK_ATTN_BNSD = 2 } sink_attn_layout;

/* The problem, passed by pointer and not retained. Checks: 0 < batch <
 * 65536; total_q, total_k, num_heads_q, num_heads_k > 0; num_heads_q %
 * num_heads_k == 0 (CANN page, axis validation); head_dim in {64, 128,
 * 256} (the page's set; 256 with bf16 or fp16 only);
 * max_seqlen_q/k equal to the true maxima of the host sequence lengths
 * (cu_seqlens differences, or seqused / S in a padded layout; the CANN page
 * leaves a mismatch undefined; here it is E_INVALID); causal in {0,1};
 * win_left, win_right >= -1; dtype a sink_attn_dtype. Layout: layout_q a
 * sink_attn_layout and layout_out equal to it, or BSND with BNSD q. TND
 * has seq_q = seq_k = 0; a padded layout has seq_q, seq_k > 0, total_q =
 * batch * seq_q and total_k = batch * seq_k (all rows, padding included).
 * A zero-initialised tail (layout TND, seq 0) is the packed problem. */
typedef struct {
  int32_t batch, num_heads_q, num_heads_k, head_dim;
  int32_t total_q, total_k, max_seqlen_q, max_seqlen_k;
  int32_t causal, win_left, win_right;
  int32_t dtype;
  int32_t layout_q, layout_out;
  int32_t seq_q, seq_k;
} sink_attn_problem;

/* Tile schedule ("CANN ops-transformer: flash_attn", Function section: a
 * separate metadata call records the task split that the main call then
 * uses). Host only, synchronous, touches no GPU.
 *
 * Reads the HOST copies of cu_seqlens_q/k ([batch+1] int32 each). Writes an
 * int32 table into meta_host (capacity meta_capacity_words) and reports
 * *meta_words (table size), *fwd_workspace_bytes and *bwd_workspace_bytes
 * (device scratch the later calls need). Two-call protocol: with
 * meta_host == NULL only the three sizes are written. The table holds a
 * header that repeats every problem field, the tile sizes, and the work
 * items: per (sequence, query tile) the range of key tiles with at least one
 * kept element and, inside it, the range whose every element is kept; the
 * same per (sequence, key tile) for the backward; and split-KV items for
 * short query groups (max_seqlen_q * num_heads_q / num_heads_k <= 64:
 * decode mode, where the forward runs them; the backward's dQ pass always
 * walks the per-query-tile items). Masked-out tiles are never visited.
 * Copy the table unchanged to device memory (meta_dev) for fwd/bwd. The
 * forward calls read only the first meta_host[SINK_ATTN_META_FWD_WORDS]
 * words of meta_dev (the header and the items the forward walks), so a
 * caller that runs no backward with the table may copy just that prefix;
 * the backward reads the whole table. The tile kernels take each sequence's
 * first rows and lengths from the table (the host cu_seqlens it was built
 * from), other kernels from the device cu_seqlens: the two copies must hold
 * the same values.
 * Errors: E_INVALID (problem or cu_seqlens checks above, NULL pointers, a
 * padded layout), E_UNSUPPORTED, E_BUFFER_TOO_SMALL (meta_capacity_words <
 * *meta_words; the sizes are still written). */
sink_attn_status sink_attn_metadata(const sink_attn_problem* p,
                                    const int32_t* cu_seqlens_q_host,
                                    const int32_t* cu_seqlens_k_host,
                                    int32_t* meta_host,
                                    int64_t meta_capacity_words,
                                    int64_t* meta_words,
                                    int64_t* fwd_workspace_bytes,
                                    int64_t* bwd_workspace_bytes);

/* Forward. Enqueues on `stream` and returns. meta_host is the table from
 * sink_attn_metadata for this same problem (its header is compared with *p:
 * E_META_MISMATCH), meta_dev its device copy. q, k, v, cu_seqlens_q/k,
 * sink_logits (may be NULL = no sink), out, lse and workspace are device
 * pointers; workspace must hold fwd_workspace_bytes (may be NULL when that
 * is 0). scale must be finite and > 0 (the Python layer defaults it to
 * 1/sqrt(head_dim), as the "slime" wrapper does). Writes out and lse.
 * Errors: E_INVALID, E_UNSUPPORTED, E_META_MISMATCH, E_BUFFER_TOO_SMALL,
 * E_HIP. */
sink_attn_status sink_attn_fwd(const sink_attn_problem* p,
                               const int32_t* meta_host,
                               const int32_t* meta_dev,
                               const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k,
                               const float* sink_logits, float scale,
                               void* out, float* lse,
                               void* workspace, int64_t workspace_bytes,
                               hipStream_t stream);

/* Backward. Same conventions as sink_attn_fwd. out and lse are what
 * sink_attn_fwd wrote for the same inputs; dout has the layout of out.
 * Writes dq, dk, dv (dtype) and dsink ([num_heads_q] fp32). dsink must be
 * NULL exactly when sink_logits is NULL. workspace must hold
 * bwd_workspace_bytes. Every output is deterministic: dq is computed by a
 * query-tile-outer pass, not accumulated with atomics.
 * Errors: as sink_attn_fwd; E_META_MISMATCH for a paged table. */
sink_attn_status sink_attn_bwd(const sink_attn_problem* p,
                               const int32_t* meta_host,
                               const int32_t* meta_dev,
                               const void* dout, const void* q, const void* k,
                               const void* v, const void* out, const float* lse,
                               const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k,
                               const float* sink_logits, float scale,
                               void* dq, void* dk, void* dv, float* dsink,
                               void* workspace, int64_t workspace_bytes,
                               hipStream_t stream);

/* Paged K/V cache: the keys and values of a sequence live in fixed-size
 * pages of one cache tensor, found through a block table ("CANN
 * ops-transformer: flash_attn", Paged Attention parameter group and the
 * PA_BBND and PA_BNBD k/v layouts; "hf-attention-normalizers",
 * Differentiable Paged Attention: the kernel reads physical pages through
 * the block table and never gathers a copy). Layouts:
 *   k_cache, v_cache : PA_BBND [num_blocks, block_size, num_heads_k, head_dim]
 *                      or PA_BNBD [num_blocks, num_heads_k, block_size,
 *                      head_dim] (dtype)
 *   block_table      : [batch, max_blocks_per_seq] int32
 *   seqused_kv       : [batch] int32, keys of sequence b
 * Key row r < seqused_kv[b] of sequence b is slot r % block_size of page
 * block_table[b][r / block_size]. Pages may be shared between sequences and
 * appear in any order. Only the forward is paged; the page's PA_NZ layout
 * (16-wide column fractals) is not taken. */
typedef enum { SINK_ATTN_PA_BBND = 0, SINK_ATTN_PA_BNBD = 1 } sink_attn_cache_layout;
typedef struct {
  int32_t block_size;          /* 16..1024 and a multiple of 16 (CANN page) */
  int32_t max_blocks_per_seq;  /* columns of block_table, > 0              */
  int32_t num_blocks;          /* pages in each cache tensor, > 0          */
  int32_t layout;              /* sink_attn_cache_layout                  */
} sink_attn_paged_kv;

/* Tile schedule for a paged forward. As sink_attn_metadata, with the key
 * lengths given as seqused_kv_host ([batch] int32; p->total_k must be their
 * sum and p->max_seqlen_k their maximum) and the HOST copy of the block
 * table, whose entries for the pages in use must lie in [0, num_blocks):
 * they are checked here and hashed into the header, and the device copy
 * passed to sink_attn_fwd_paged must equal it (not checked there). Short
 * query groups (max_seqlen_q * num_heads_q / num_heads_k <= 64) run the
 * split-KV decode path, longer ones the tiled prefill path (a chunked
 * prefill against the cache); bf16 or fp16 only (fp32: E_UNSUPPORTED). The
 * table can only be used with sink_attn_fwd_paged: it holds no backward
 * items, and in decode mode no per-query-tile items.
 * Errors: E_INVALID, E_UNSUPPORTED, E_BUFFER_TOO_SMALL. */
sink_attn_status sink_attn_metadata_paged(const sink_attn_problem* p,
                                          const sink_attn_paged_kv* kv,
                                          const int32_t* cu_seqlens_q_host,
                                          const int32_t* seqused_kv_host,
                                          const int32_t* block_table_host,
                                          int32_t* meta_host,
                                          int64_t meta_capacity_words,
                                          int64_t* meta_words,
                                          int64_t* fwd_workspace_bytes);

/* Paged forward. As sink_attn_fwd, with k_cache, v_cache, block_table and
 * seqused_kv (device pointers, layouts above) in place of k, v and
 * cu_seqlens_k. meta_host must come from sink_attn_metadata_paged for this
 * problem and this *kv (E_META_MISMATCH otherwise). The results equal those
 * of sink_attn_fwd on the gathered contiguous keys and values, bit for bit.
 * Errors: as sink_attn_fwd. */
sink_attn_status sink_attn_fwd_paged(const sink_attn_problem* p,
                                     const sink_attn_paged_kv* kv,
                                     const int32_t* meta_host,
                                     const int32_t* meta_dev, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* block_table,
                                     const int32_t* cu_seqlens_q,
                                     const int32_t* seqused_kv,
                                     const float* sink_logits, float scale,
                                     void* out, float* lse, void* workspace,
                                     int64_t workspace_bytes,
                                     hipStream_t stream);

/* Batch-padded layouts (BSND, BNSD; CANN page, q, k, v validation, the
 * layout matching table and the SeqLengths parameter group): every
 * sequence owns seq_q query rows and seq_k key rows of the tensors, of which
 * the first seqused_q[b] / seqused_kv[b] are in use (all of them when the
 * pointer is NULL). The method, the masks (bottom-right alignment over the
 * used lengths) and the results on the used rows are those of the packed
 * calls on the same sequences. cu_seqlens play no part.
 *
 * Metadata: as sink_attn_metadata, from the HOST copies of seqused_q /
 * seqused_kv ([batch] int32 each, NULL = S for every sequence). Whether each
 * pointer was NULL is recorded in the header; the device pointers passed to
 * the calls below must match (E_META_MISMATCH). A table made here is for
 * sink_attn_fwd_padded / sink_attn_bwd_padded only.
 * Errors: E_INVALID (problem checks, a TND layout, used lengths outside
 * [0, S]), E_UNSUPPORTED, E_BUFFER_TOO_SMALL. */
sink_attn_status sink_attn_metadata_padded(const sink_attn_problem* p,
                                           const int32_t* seqused_q_host,
                                           const int32_t* seqused_kv_host,
                                           int32_t* meta_host,
                                           int64_t meta_capacity_words,
                                           int64_t* meta_words,
                                           int64_t* fwd_workspace_bytes,
                                           int64_t* bwd_workspace_bytes);

/* Forward over a padded layout. As sink_attn_fwd, with the device copies of
 * seqused_q / seqused_kv (or NULL, as for the metadata) in place of
 * cu_seqlens_q/k; tensors in the layouts above. Writes out and lse on the
 * used rows only.
 * Errors: as sink_attn_fwd. */
sink_attn_status sink_attn_fwd_padded(const sink_attn_problem* p,
                                      const int32_t* meta_host,
                                      const int32_t* meta_dev,
                                      const void* q, const void* k, const void* v,
                                      const int32_t* seqused_q,
                                      const int32_t* seqused_kv,
                                      const float* sink_logits, float scale,
                                      void* out, float* lse,
                                      void* workspace, int64_t workspace_bytes,
                                      hipStream_t stream);

/* Backward over a padded layout. As sink_attn_bwd, with seqused_q /
 * seqused_kv as for sink_attn_fwd_padded; dout has out's layout
 * (layout_out), dq q's, dk and dv k's. Writes dq, dk, dv on the used rows
 * only, and dsink. Deterministic.
 * Errors: as sink_attn_bwd. */
sink_attn_status sink_attn_bwd_padded(const sink_attn_problem* p,
                                      const int32_t* meta_host,
                                      const int32_t* meta_dev,
                                      const void* dout, const void* q, const void* k,
                                      const void* v, const void* out, const float* lse,
                                      const int32_t* seqused_q,
                                      const int32_t* seqused_kv,
                                      const float* sink_logits, float scale,
                                      void* dq, void* dk, void* dv, float* dsink,
                                      void* workspace, int64_t workspace_bytes,
                                      hipStream_t stream);

/* Bytes of the device array behind sink_attn_bwd_noalloc (64 MiB). */
#define SINK_ATTN_NOALLOC_SCRATCH_BYTES (64LL << 20)

/* Backward that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Arguments, results and
 * errors as sink_attn_bwd (TND layout), without workspace and
 * workspace_bytes. Its scratch (the row terms D and the dsink partials,
 * bwd_workspace_bytes of the metadata: about 4 * num_heads_q * total_q
 * bytes) lives in a static device array of SINK_ATTN_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends;
 * its address is looked up once per device, on the first call with that
 * device current. The current device must be the one `stream` belongs to.
 * Every call on a GPU shares that GPU's array: calls that overlap on one
 * GPU (on two streams, or two host threads) race and give wrong results;
 * calls ordered on one stream are safe. The kernels write every scratch
 * word before reading it, so nothing is cleared between calls. Under HIP
 * graph capture, make the first call on a device before capturing (the
 * address lookup is not a stream operation); the call itself enqueues
 * kernel launches only.
 * Errors: as sink_attn_bwd; E_BUFFER_TOO_SMALL when the metadata's
 * bwd_workspace_bytes exceed SINK_ATTN_NOALLOC_SCRATCH_BYTES; E_HIP when
 * the array's address cannot be obtained. */
sink_attn_status sink_attn_bwd_noalloc(const sink_attn_problem* p,
                                       const int32_t* meta_host,
                                       const int32_t* meta_dev,
                                       const void* dout, const void* q, const void* k,
                                       const void* v, const void* out, const float* lse,
                                       const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_k,
                                       const float* sink_logits, float scale,
                                       void* dq, void* dk, void* dv, float* dsink,
                                       hipStream_t stream);

/* Context-parallel merge. "CANN ops-transformer: flash_attn", Note on
 * softmax_lse: ring attention combines partial results through their lse.
 * Each of num_parts partials is the attention of the same queries over a
 * disjoint part of the keys, computed WITHOUT the sink (sink_logits NULL):
 * its output out_p and its lse_p = ln sum e^S over that part. The merge
 * returns the attention over the union of the parts with the sink added
 * exactly once:
 *   lse = ln(e^{s_h} + sum_p e^{lse_p}),  out = sum_p e^{lse_p - lse} out_p.
 * Parts with lse_p = -inf (no kept key) contribute nothing. Layouts (device
 * pointers, contiguous): partial_out [num_parts, total_q, num_heads_q,
 * head_dim] in part_dtype (16-byte aligned); partial_lse [num_parts,
 * num_heads_q, total_q] fp32; sink_logits [num_heads_q] fp32 or NULL; out
 * [total_q, num_heads_q, head_dim] in out_dtype (16-byte aligned); lse
 * [num_heads_q, total_q] fp32, sink inclusive. Arithmetic is fp32; a bf16
 * part_dtype adds that rounding of each partial to the result. Enqueues on
 * `stream`; allocates nothing. Errors: E_INVALID (num_parts outside
 * [1, 4096], total_q or num_heads_q <= 0, NULL or misaligned pointers),
 * E_UNSUPPORTED (head_dim not 64, 128 or 256, unknown dtype, more than 2^40
 * elements), E_HIP. */
sink_attn_status sink_attn_merge(int32_t num_parts, int32_t total_q,
                                 int32_t num_heads_q, int32_t head_dim,
                                 int32_t part_dtype, int32_t out_dtype,
                                 const void* partial_out,
                                 const float* partial_lse,
                                 const float* sink_logits, void* out,
                                 float* lse, hipStream_t stream);

/* Copies `words` int32 of a metadata table from pinned host memory to device
 * memory with a kernel on `stream` (the GPU reads the pinned pages
 * directly), instead of a copy on a DMA engine. The kernels that read the
 * table next in the same stream then depend only on an earlier kernel of
 * their own queue; a DMA-engine copy between two attention calls costs a
 * cross-engine wait of tens of microseconds, which at decode shapes (one
 * call every millisecond) is several percent of the step. The two-phase
 * metadata model of "CANN ops-transformer: flash_attn" (Function section)
 * leaves this upload to the caller; this is one way to do it.
 * host: allocated with hipHostMalloc (torch's pin_memory()); it is read when
 * the kernel runs, so it must not change before that (stream order).
 * dev: device memory of at least `words` int32, not overlapping host.
 * Errors: E_INVALID (NULL pointers, words < 0, host not pinned host memory,
 * dev not device memory), E_HIP. words = 0 enqueues nothing. */
sink_attn_status sink_attn_upload_table(const int32_t* host, int32_t* dev, int64_t words,
                                        hipStream_t stream);

/* Measurement aid: the next sink_attn_fwd or sink_attn_bwd made on this host
 * thread records `start` just before and `stop` just after its main kernel
 * (forward: the attention tile loop, or the split-KV kernel for short query
 * groups; backward: the dK/dV tile loop), on its stream, and then disarms.
 * sink_attn_fwd_paged counts as a forward, sink_attn_merge records around
 * its merge kernel. Pass NULL, NULL to disarm. The events belong to the
 * caller. */
sink_attn_status sink_attn_arm_timing(hipEvent_t start, hipEvent_t stop);

/* Static text for a status code. */
const char* sink_attn_status_string(sink_attn_status s);

/* SINK_ATTN_ABI_VERSION of the built library. */
int32_t sink_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SINK_ATTN_H */
