/*
 * bvf.h -- C ABI of the MI355X (gfx950) batched verify forward for DFlash block speculative decoding.
 *
 * What the library computes (sources are web pages, cited by title and section):
 *   [PR2303] engine PR #2303 "npu forward: Gemma4 verifies a draft in one batched pass; KV row width
 *            per layer": the batched body runs all k drafted rows through every layer in one pass over
 *            the weights ("What changes"); a KV-shared layer reads its owner's cache and appends
 *            nothing; every row's logits are returned; KV row width is per layer (item 1);
 *            commit_verify_rows keeps n of the k verified rows ("Proof": 3 + 2 = 5 positions held).
 *   [CARD]   "FastFlowLM build: Nemotron-3.5-Bolt-E4B-DFlash-NPU2": Q4_1 weights (32-weight blocks,
 *            scale + minimum, 5 bits per weight; "Weights" row), the draft's geometry ("Draft" row),
 *            its taps ("Taps" row), the greedy longest-prefix accept ("How it is used").
 *   [PR2236] engine PR #2236 "npu: a Gemma4 pack stops re-reading its weights every token;
 *            tools/dflash_acceptance": weights packed once at load (section 1); the draft block
 *            [token s, mask, ...] over tapped context rows, rows >= 1 through the target head
 *            (section 2, the acceptance tool's header).
 *
 * Conventions
 *   - Every pointer named d_* is device memory on the model's device; h_* is host memory. The caller
 *     owns every pointer it passes. Host inputs are copied before the call returns.
 *   - All device work is enqueued on the stream given at bvf_create; outputs are valid once that
 *     stream has been synchronised. Calls on one model must not overlap (one stream, one caller).
 *   - Every call validates its arguments and the model state before it enqueues anything: a
 *     non-zero status means nothing was enqueued and no state changed. bvf_last_error() returns a
 *     thread-local message for the last failing call on this thread.
 *   - Numbers: residual stream fp32; GEMM inputs bf16 (round to nearest even); GEMM accumulation and
 *     outputs fp32; K/V planes fp32; logits fp32; Q4_1 weights are dequantised exactly.
 */
#ifndef BVF_H
#define BVF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BVF_OK = 0,
    BVF_E_INVALID = 1,   /* an argument is out of range or inconsistent with the model */
    BVF_E_STATE = 2,     /* the call does not fit the model's state (e.g. commit with no verify) */
    BVF_E_CAPACITY = 3,  /* positions would exceed max_ctx, or a buffer is too small */
    BVF_E_DEVICE = 4     /* a HIP runtime call failed */
} bvf_status;

enum { BVF_ATTN_SLIDING = 0, BVF_ATTN_FULL = 1 };

/* Q4_1 matrices of a layer. The library fuses Q|K|V into one packed matrix and interleaves GATE and
 * UP by 16-column tiles; each load call fills its part of the packed image. */
enum { BVF_Q = 0, BVF_K = 1, BVF_V = 2, BVF_O = 3, BVF_GATE = 4, BVF_UP = 5, BVF_DOWN = 6,
       BVF_PLE_GATE = 7,   /* per-layer embedding gate [ple_dim][hidden] (models with ple_dim > 0) */
       BVF_PLE_PROJ = 8 }; /* per-layer embedding projection [hidden][ple_dim] */

/* bf16 tensors. */
enum {
    BVF_EMBED = 0,       /* [vocab][hidden]: tied embedding table and output head (target only) */
    BVF_FINAL_NORM = 1,  /* [hidden] */
    BVF_ATTN_NORM = 2,   /* per layer [hidden] */
    BVF_MLP_NORM = 3,    /* per layer [hidden] */
    BVF_Q_NORM = 4,      /* per layer [head_dim] */
    BVF_K_NORM = 5,      /* per layer [head_dim] */
    BVF_FC = 6,          /* draft only: [hidden][n_taps * hidden], fuses the tapped target rows */
    BVF_HIDDEN_NORM = 7, /* draft only: [hidden], RMSNorm gain applied after fc */
    BVF_PLE_TABLE = 8,   /* ple_dim > 0: [vocab][n_layers * ple_dim] per-layer inputs, row = token id */
    BVF_LAYER_SCALAR = 9 /* ple_dim > 0: per layer [1], the factor applied to the layer's output */
};

typedef struct {
    int32_t attn;        /* BVF_ATTN_SLIDING or BVF_ATTN_FULL */
    int32_t n_kv_heads;  /* KV row width of the layer w = n_kv_heads * head_dim floats (K; V the same) */
    int32_t head_dim;    /* multiple of 64, <= 256 */
    int32_t window;      /* sliding layer: a row at position p sees keys [p - window + 1, p]; 0 = all */
    int32_t ffn;         /* SwiGLU width */
    int32_t kv_owner;    /* -1: the layer holds its own KV plane. Else the index of an earlier own
                            layer of the same attention type and geometry whose plane it reads; the
                            layer then has no K/V projection and appends nothing [PR2303]. */
} bvf_layer_desc;

typedef struct {
    int32_t n_layers;
    int32_t hidden;        /* multiple of 128 */
    int32_t n_q_heads;     /* multiple of every layer's n_kv_heads */
    int32_t vocab;         /* target: rows of the embedding/head table; draft: 0 */
    int32_t max_ctx;       /* plane capacity in positions (cached context + rows in flight) */
    int32_t qk_norm;       /* 1: per-head RMSNorm on q and k before RoPE */
    int32_t block_causal;  /* 1: a verify model (rows causal, appended to the planes);
                              0: a DFlash draft (block rows see each other and the context) */
    int32_t draft_window;  /* draft: the block sees the last draft_window context rows; 0 = all */
    int32_t n_taps;        /* target: layers whose outputs are tapped; draft: taps fused by fc */
    const int32_t* tap_layers; /* target: n_taps zero-based layer ids, written in this order */
    float rope_base;       /* rotate-half RoPE, pairs (i, i + head_dim/2), angle p * base^(-2i/hd) */
    float rms_eps;         /* RMSNorm: x / sqrt(mean(x^2) + eps) * gain */
    const bvf_layer_desc* layers;
    int32_t kv_bf16;       /* 0: K/V planes hold fp32 values (the pages' floats); 1: a memory variant
                              holding bf16 values, every stored K/V value (cached by bvf_set_kv, appended
                              by a pass, or a draft block's own rows) rounded from fp32 to nearest even.
                              Counts (plane_floats, cut_floats) are in values either way. */
    int32_t ple_dim;       /* 0, or the per-layer embedding width (multiple of 128, verify models only).
                              After its MLP every layer runs the PLE tail [PR2303, "What changes": the
                              per-layer inputs of every row, the PLE gate and projection as M-row GEMMs,
                              then the layer scalar]: u = Wg . bf16(x) [ple_dim], h = bf16(silu(u) * p)
                              with p = row l of the per-layer input table entry of the row's token,
                              x = (x + Wp . h) * s_l. The per-layer inputs need token ids, so calls that
                              take injected rows (bvf_layer_forward) are refused on such a model. */
    int32_t kv_ring;       /* 0: linear planes (every position held). 1: a memory variant for verify
                              models: each own sliding layer with a window keeps a ring of window + 16
                              position slots, position p in slot p mod (window + 16); the 16 spare
                              slots take a pass's rows, so rows a commit cuts back never overwrite a
                              key that a later row can see. Such a plane holds, counts, snapshots and
                              returns (bvf_get_kv) the last min(held, window) positions; older rows
                              read as NaN. Cuts stay per layer [PR2303, "What changes" item 1]. */
} bvf_model_desc;

typedef struct bvf_model bvf_model;
typedef struct bvf_snapshot bvf_snapshot;

/* Thread-local message of the last failing call ("" if none). Never NULL. */
const char* bvf_last_error(void);

/* Device bytes the caller must provide to bvf_create for this descriptor (weights, KV planes,
 * activations and scratch; 256-byte aligned). Returns 0 and sets the error for an invalid
 * descriptor. No device call is made. */
size_t bvf_arena_bytes(const bvf_model_desc* desc);

/* Create a model inside the caller's device arena (at least bvf_arena_bytes(desc) bytes, 256-byte
 * aligned, on the current device). hip_stream: the hipStream_t all work is enqueued on (NULL = the
 * null stream). The arena is zero-filled; the descriptor is copied. */
bvf_status bvf_create(const bvf_model_desc* desc, void* d_arena, size_t arena_bytes, void* hip_stream,
                      bvf_model** out);
void bvf_destroy(bvf_model* m);

/* Load one Q4_1 matrix of a layer from its canonical host image (packed once; [PR2236] section 1):
 * n_out rows of n_in/32 blocks of 20 bytes {fp16 scale, fp16 min, 16 code bytes}; code j < 16 in the
 * low nibble of byte j, code j + 16 in the high nibble; weight = scale * code + min ([CARD],
 * "Weights" row). n_in must be the matrix's input width (a multiple of 128), n_out its output width.
 * BVF_K / BVF_V on a KV-shared layer are refused. */
bvf_status bvf_load_q4_1(bvf_model* m, int32_t layer, int32_t matrix, const void* h_blocks, size_t bytes,
                         int32_t n_out, int32_t n_in);

/* Load a bf16 tensor (see the enum for shapes; layer ignored for model-wide tensors). n = elements. */
bvf_status bvf_load_bf16(bvf_model* m, int32_t tensor, int32_t layer, const uint16_t* h, size_t n);

/* Cached context of an own plane: h_kv [positions][2][w] fp32 (K then V per position, K already
 * normalised and rotated). The same `positions` must be set on every own plane before a verify;
 * bvf_set_positions then fixes the count. Refused on a shared layer. */
bvf_status bvf_set_kv(bvf_model* m, int32_t layer, const float* h_kv, int64_t positions);
bvf_status bvf_set_positions(bvf_model* m, int64_t positions);
/* extend_context [PR2303, "What changes" item 1: it is one of the operations whose KV count is per
 * layer]: appends n positions of given K/V rows to every own plane at the held count, each at that
 * layer's own width w_l, and positions held += n; shared planes stay empty. h_kv_all (host, read
 * before the call returns) holds the own layers' new rows one after the other in layer order, each
 * [n][2][w_l] fp32 (K then V per position, K already normalised and rotated, as for bvf_set_kv);
 * bf16 planes store each value rounded to nearest even. Synchronous with the model's stream.
 * Refused with no state change: a verify pending (BVF_E_STATE), held + n > max_ctx
 * (BVF_E_CAPACITY), n < 0 or h_kv_all NULL with n > 0 (BVF_E_INVALID). n = 0 does nothing. */
bvf_status bvf_extend_context(bvf_model* m, const float* h_kv_all, int64_t n);
/* Read back the first `positions` rows of an own plane into h_kv [positions][2][w] fp32, in the
 * layout bvf_set_kv takes (bf16 planes are widened exactly). Waits for the model's stream. Rows at
 * or beyond the held count hold whatever the last pass or set_kv left there. Refused on a shared
 * layer; positions > max_ctx is BVF_E_CAPACITY. */
bvf_status bvf_get_kv(const bvf_model* m, int32_t layer, float* h_kv, int64_t positions);


/* Per-layer KV bookkeeping [PR2303, "What changes" item 1]. kv_widths: w of each layer (a shared
 * layer reports its owner's width). plane_floats: floats held by each layer's own plane (held
 * positions x 2 x w; 0 on a shared layer). positions_held: positions held (same on every own plane).
 * n must equal n_layers. */
bvf_status bvf_kv_widths(const bvf_model* m, int64_t* h_out, int32_t n);
bvf_status bvf_plane_floats(const bvf_model* m, int64_t* h_out, int32_t n);
bvf_status bvf_positions_held(const bvf_model* m, int64_t* h_out);

/* The batched verify [PR2303, "What changes"]: rows d_tokens[0..k) at positions P..P+k-1
 * (P = positions held) go through every layer in one pass over the packed weights; a KV-shared layer
 * reads its owner's plane. Writes every row's logits, d_logits_all [k][vocab] fp32, and, if d_taps is
 * not NULL, the tapped layer outputs d_taps [k][n_taps][hidden] bf16. Appends k rows to every own
 * plane (positions held = P + k) until bvf_commit_verify_rows cuts them back. 1 <= k <= 16. */
bvf_status bvf_verify_batch(bvf_model* m, const int32_t* d_tokens, int32_t k, float* d_logits_all,
                            uint16_t* d_taps);

/* Chunked prefill ([PR2303] "What changes": the batched body; "Proof": the state test's chunk arms):
 * the n tokens d_tokens[0..n) at positions P .. P+n-1 (P = positions held) go through every layer
 * in chunks of up to 64 rows, each chunk one batched pass over the packed weights (every weight
 * superblock feeds up to four 16-row MFMA tiles), and are kept (positions held = P + n; no commit
 * needed). The head runs once, on the last row; d_last_logits [vocab] fp32 (NULL allowed) receives
 * that row's logits. With bvf_snapshot_take /
 * bvf_restore this is a prefix cache: prefill a shared prefix once, snapshot, and restore it before
 * each continuation. Refuses n < 1 (BVF_E_INVALID), P + n > max_ctx (BVF_E_CAPACITY) and a pending
 * verify (BVF_E_STATE: commit it first); a refusal changes nothing. */
bvf_status bvf_prefill(bvf_model* m, const int32_t* d_tokens, int32_t n, float* d_last_logits);

/* Graph replay (1) or direct launches (0, the default) of bvf_verify_batch on a verify model and of
 * bvf_draft_block_forward with a block on a draft model. With 1 the pass is captured into a HIP graph
 * (on a private stream) and replayed on the model's stream; the replayed pass reads the positions
 * held from device memory (set by a one-thread kernel launched before each replay).
 * Verify: the capture serves every position of a 256-position span (P with the same P / 256, below
 * max_ctx - k) while k and the three buffer pointers stay the same; it is taken again when any of
 * them changes. Both modes plan the attention for the span's last position, so their results are
 * identical bit for bit.
 * Draft: one capture per context-row count n_new (0 .. 16), kept while the layers' attention plans
 * at the current positions (constant once the context window is full), the block size, the
 * embedding scale, the mask token, the target model and the four buffer pointers stay the same.
 * A replay runs the launches of the direct path with the same plans, so the results are identical
 * bit for bit. The append-only call (block 0) always launches directly. */
bvf_status bvf_set_graph_mode(bvf_model* m, int32_t on);
/* Number of graph captures the model has taken so far (h_out[0]): verify passes on a verify model,
 * draft blocks on a draft model. */
bvf_status bvf_graph_captures(const bvf_model* m, int64_t* h_out);

/* Greedy longest-prefix accept ([CARD], "How it is used"; [PR2236], the acceptance tool): y_i is the
 * first index of the maximum of row i of d_logits_all [k][vocab] (NaN never wins); the drafts are
 * d_tokens[1..k); a = the largest j <= k-1 with d_tokens[m] == y_{m-1} for all 1 <= m <= j. Writes
 * d_out_tokens[0..a] = d_tokens[1..a], y_a (the a accepted drafts and the target's own token), and
 * d_n_accepted[0] = a. Device outputs; no host synchronisation. */
bvf_status bvf_accept_greedy(bvf_model* m, const float* d_logits_all, int32_t k, const int32_t* d_tokens,
                             int32_t* d_out_tokens, int32_t* d_n_accepted);

/* The greedy accept of bvf_accept_greedy without a model and without any allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). d_logits_all [k][vocab] fp32, d_tokens [k], d_out_tokens [k] and
 * d_n_accepted [1] are device buffers the caller owns; the work is enqueued on hip_stream (NULL:
 * the null stream). The argmax partials live in a fixed device array of the library, one per GPU
 * (16 x 256 x 8 bytes, held until the process ends): k <= 16 and vocab <= 1048576, else
 * BVF_E_INVALID / BVF_E_CAPACITY before anything is enqueued. The first call on a device looks up
 * that device's array (the device must be current). Calls on one GPU share the array: calls that
 * overlap on one GPU (other streams, other threads) race; calls on one stream do not. */
bvf_status bvf_accept_greedy_static(const float* d_logits_all, int32_t k, int32_t vocab, const int32_t* d_tokens,
                                    int32_t* d_out_tokens, int32_t* d_n_accepted, void* hip_stream);

/* Sampled accept at temperature T > 0 ([CARD], "How it is used": with a sampler every position is
 * sampled and compared with the draft, so the output follows the target's distribution). Row i's
 * draw y_i is the first index of the maximum of fmaf(z_ij, 1/T, -log(-log u_ij)) in fp32 (the
 * Gumbel-max method: y_i follows softmax(z_i / T)); u_ij = ((x >> 9) + 1/2) / 2^23 where x is the word
 * j % 4 of the Philox4x32-10 block (Salmon, Moraes, Dror, Shaw, SC 2011) at counter
 * (j / 4, i, offset bits 0-31, offset bits 32-63) under key (seed bits 0-31, seed bits 32-63). The accept
 * then runs as in bvf_accept_greedy with y in place of the argmax. d_draws (NULL allowed) receives
 * y [k]. The same (logits, seed, offset) always give the same draws; callers advance offset per call.
 * Refuses a temperature that is not finite or not > 0 (BVF_E_INVALID). Device outputs; no host
 * synchronisation. */
bvf_status bvf_accept_sampled(bvf_model* m, const float* d_logits_all, int32_t k, const int32_t* d_tokens,
                              float temperature, uint64_t seed, uint64_t offset, int32_t* d_out_tokens,
                              int32_t* d_n_accepted, int32_t* d_draws);

/* Harness hook for seeded acceptance (not part of the method): d_logits_all[i][d_tok[i]] += d_add[i]. */
bvf_status bvf_steer_logits(bvf_model* m, float* d_logits_all, int32_t k, const int32_t* d_tok,
                            const float* d_add);

/* Keep n (0 <= n <= k) of the k rows of the last verify on every own plane: positions held becomes
 * P + n; shared planes stay empty [PR2303, "What changes" item 1, "Proof"]. Moves no data. Refused
 * with BVF_E_STATE if no verify is pending or n > k. */
bvf_status bvf_commit_verify_rows(bvf_model* m, int32_t n);

/* Snapshot / restore of the held prefix of every own plane at its own width; shared planes stay
 * empty [PR2303, "What changes" item 1]. The library allocates and owns the snapshot's device copy
 * until bvf_snapshot_free. A snapshot is of committed state: snapshot_take is refused with
 * BVF_E_STATE (no state change) while a verify is pending, and leaves the model unchanged
 * otherwise. Restore refuses a snapshot whose layer count or widths differ, and clears a pending
 * verify. snapshot_floats: floats kept per layer (0 on shared layers). */
bvf_status bvf_snapshot_take(bvf_model* m, bvf_snapshot** out);
/* Re-take a snapshot of the model's committed state into an existing snapshot of the same model
 * shape (layers, widths, plane capacities, stored element size), allocating nothing: each own
 * plane's kept rows must fit the rows the snapshot was first taken with, else BVF_E_CAPACITY; a
 * pending verify is BVF_E_STATE; a shape mismatch BVF_E_INVALID. A refusal leaves the snapshot
 * unchanged. For prefix caches that refresh their snapshot (a snapshot taken at the largest state
 * holds any smaller one). */
bvf_status bvf_snapshot_update(bvf_model* m, bvf_snapshot* s);
bvf_status bvf_restore(bvf_model* m, const bvf_snapshot* s);
bvf_status bvf_snapshot_floats(const bvf_snapshot* s, int64_t* h_out, int32_t n);
void bvf_snapshot_free(bvf_snapshot* s);

/* DFlash draft block forward ([CARD] "Draft", "Taps", "How it is used"; [PR2236] section 2):
 * appends n_new context rows from their taps d_new_taps [n_new][n_taps][hidden] bf16 (fc, then
 * RMSNorm with the hidden-norm gain, then K/V in every draft layer at positions s - n_new .. s - 1,
 * s = the draft's new positions held), runs the block [d_last_token[0], mask x (block - 1)] (target
 * embeddings times embedding_scale, positions s .. s + block - 1; rows see each other and the last
 * draft_window context rows), the final norm, the target's head on rows 1 .. block-1 and writes their
 * argmax to d_proposals [block - 1]. d_logits (optional) receives those rows' logits [block-1][vocab].
 * 2 <= block <= 16, 0 <= n_new, n_new + block <= 16. block = 0 only appends the n_new (<= 16)
 * context rows (prefill of the draft context); d_last_token and d_proposals may then be NULL. */
bvf_status bvf_draft_block_forward(bvf_model* draft, const bvf_model* target, const uint16_t* d_new_taps,
                                   int32_t n_new, const int32_t* d_last_token, int32_t block,
                                   float embedding_scale, int32_t mask_token, int32_t* d_proposals,
                                   float* d_logits);

/* Kernel-level entry points (parity tests and measurement). */
/* Dequantised fp32 weights of one loaded Q4_1 matrix, d_w [n_out][n_in]. */
bvf_status bvf_q4_1_dequant(const bvf_model* m, int32_t layer, int32_t matrix, float* d_w);
/* d_y [rows][n_out] fp32 = d_x [rows][n_in] bf16 times the matrix (the fused-matrix kernel, run on
 * the one matrix's columns; GATE and UP give their own halves). 1 <= rows <= 16 on a draft, <= 64 on
 * a verify model (the prefill chunk width: 17..64 rows take the kernel's 2 or 4 row-tile form). */
bvf_status bvf_q4_1_gemm(const bvf_model* m, int32_t layer, int32_t matrix, const uint16_t* d_x, int32_t rows,
                         float* d_y);
/* One verify layer (the kernels of bvf_verify_batch) over d_x [rows][hidden] fp32, in place, at
 * positions P .. P + rows - 1 (P = positions held), 1 <= rows <= 64. An own layer writes its K/V rows
 * into its plane at those positions; the positions held do not change. For layer-by-layer parity
 * tests. */
bvf_status bvf_layer_forward(bvf_model* m, int32_t layer, float* d_x, int32_t rows);
/* Measurement: launches each GEMM class of the verify pass exactly as the pass does (same kernels,
 * plans and epilogues, into the model's scratch) for every layer, `iters` times, between two HIP
 * events recorded on the model's stream, and synchronises. Class 0 = fused q|k|v, 1 = o (+residual),
 * 2 = gate|up (+SwiGLU), 3 = down (+residual), 4 = the bf16 head. h_ms[5]: average milliseconds per
 * launch; h_bytes[5]: average weight bytes streamed per launch. 1 <= rows <= 64; above 16 rows (the
 * prefill chunk widths) the head is not run and class 4 reports 0, and classes 0 and 2 stage the bf16
 * rows that the pass's own RMSNorm kernel writes (that kernel is not timed). Overwrites the scratch
 * activations. */
bvf_status bvf_time_gemms(bvf_model* m, int32_t rows, int32_t iters, float* h_ms, int64_t* h_bytes);
/* Q4_1 bytes (packed image: 5 bits per weight) and bf16 head bytes one verify pass streams. */
bvf_status bvf_pass_bytes(const bvf_model* m, int64_t* h_q4_1_bytes, int64_t* h_head_bytes);

/* Host-only KV-plane arithmetic, exported for CPU tests of the state rules (no device call):
 * floats of plane `plane` cut at `positions` with the per-plane width list per[0..n_per): plane i
 * uses per[i], a plane past the end of the list uses per[n_per - 1] [PR2303, review
 * "VERDICT at 4d10370: READY"]. Returns -1 for n_per < 1. */
int64_t bvf_cut_floats(const int64_t* per, int32_t n_per, int32_t plane, int64_t positions);

#ifdef __cplusplus
}
#endif
#endif /* BVF_H */
