// Internal interface between the C ABI (bvf_api.cpp) and the gfx950 kernels (*.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace bvf {

constexpr int kMaxRows = 16;      // k <= 16 rows per pass: one 16-row MFMA tile
constexpr int kMaxGemmRows = 64;  // prefill chunks: up to 4 row tiles share each weight pass
// row tiles of 16 the GEMM kernel runs for M rows: 1, 2 or 4
constexpr int gemm_row_tiles(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }
constexpr int kTile = 16;         // output columns per MFMA tile
constexpr int kSuper = 128;       // K per superblock = 4 Q4_1 blocks of 32
constexpr int kAttnMaxChunks = 256;   // key chunks per (query tile, KV head) merged by the combine
// floats per query vector in an attention chunk partial: hd values of O, the running maximum and
// sum, padded so every row starts 16-byte aligned
__host__ __device__ constexpr int attn_part_ld(int hd) { return hd + 4; }

// A packed Q4_1 (or bf16) weight image, column-tiled for the small-M GEMM.
//   Q4_1: codes  [n_tiles][G][64 lanes][4 x u32]: lane = sub * 16 + c holds, for block j of the
//                superblock, the 8 codes of column c at k = 128 g + 32 j + 8 sub + e (e = 0..7),
//                nibble (e >> 1) + 4 (e & 1) of dword j (so (w >> 4i) & 0x000F000F gives the pair
//                (e = 2i, 2i + 1) in the low/high halves).
//         sm     [n_tiles][G][16 columns][4 x u32]: dword j = fp16 scale | fp16 min << 16.
//         A gate|up image interleaves by half tiles: tile t holds gate rows 8t..8t+7 in columns
//         0..7 and up rows 8t..8t+7 in columns 8..15.
//   BF16: codes points at a row-major bf16 [N][K] matrix; sm unused.
struct WMat {
    const uint8_t* codes = nullptr;
    const uint8_t* sm = nullptr;
    int n_tiles = 0;   // 16-column tiles of the packed (fused) image
    int G = 0;         // K / 128
    int K = 0;
};

enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_PLE = 3 };
enum WFmt : int { W_Q4_1 = 0, W_BF16 = 1 };

// One GEMM launch: y[m][n] (+)= sum_k A[m][k] W[n][k] over the tiles tile0 + i * tile_stride,
// i = 0 .. n_run_tiles - 1; output column of tile i is 16 i + c.
struct GemmLaunch {
    WMat w;
    int fmt = W_Q4_1;
    int epi = EPI_STORE;
    int tile0 = 0, tile_stride = 1, n_run_tiles = 0;
    const uint16_t* A = nullptr;
    int lda = 0;
    int M = 0;
    float* y = nullptr;          // STORE: y[m * ldy + n]; RESID: y[m * ldy + n] += ...
    int ldy = 0;
    uint16_t* out = nullptr;     // SWIGLU: out[m * ldo + n_half] bf16
    int ldo = 0;
    uint16_t* taps = nullptr;    // RESID: optional bf16 copy of the updated rows, taps[m * ldt + n]
    int ldt = 0;
    float* partial = nullptr;    // split-K scratch
    size_t partial_floats = 0;
    int* counters = nullptr;     // split-K arrival counters (zero between launches)
    int n_counters = 0;
    int half = -1;               // STORE on a gate|up image: -1 all columns, 0 gate, 1 up
    // RMSNorm folded into the A staging: A = bf16(xsrc * rinv * gain), rinv from ss_in [M][n_ss];
    // with n_fold in 1 .. M - 1 only rows < n_fold are, and rows n_fold .. M - 1 are copied from A
    const float* xsrc = nullptr;
    int n_fold = 0;              // 0: every row (when xsrc is set)
    int ldx = 0;
    const float* ss_in = nullptr;
    int n_ss = 0;
    const uint16_t* gain = nullptr;
    float eps = 0.f;
    float* ss_out = nullptr;     // STORE/RESID: per (row, output tile) sums of squares [M][n_run_tiles]
    const uint16_t* rscale = nullptr;   // RESID: y = (y + W.A) * bf16 scalar (nullptr: no scale)
    // PLE: out[m * ldo + n] = bf16(silu(W.A) * bf16 ple[clamp(tokens[m]) * ple_ld + n])
    const int32_t* tokens = nullptr;
    const uint16_t* ple = nullptr;
    int ple_ld = 0;
    int vocab = 0;
    int n_cu = 0;                // compute units of the device (0: 256)
    int force_S = 0, force_R = 0, force_ipw = 0, force_W = 0, force_KS = 0;   // a fixed plan (all > 0), else the planner's
};

struct GemmPlan {
    int S;              // K splits (-1: no plan fits)
    int sb_per_split;   // superblocks of 128 K per split
    int waves;          // waves per workgroup (4, 8 or 16)
    int KS;             // K parts per tile inside a workgroup (summed in LDS)
    int R;              // weight ring depth per wave (superblocks in flight)
    int ring_slots;     // LDS slots per ring (R)
    int grid;           // workgroups (all resident at once)
    size_t lds;         // dynamic LDS bytes: weight rings, block sums, activation rows
};
constexpr size_t kLdsPerCu = 160 * 1024;            // gfx950 LDS per compute unit
constexpr size_t kGemmLdsMax = 160 * 1024 - 1024;   // per workgroup (static LDS sits beside it)

size_t gemm_lds_bytes(int fmt, int M, int sb, int waves, int ring, int KS);

GemmPlan plan_gemm(const GemmLaunch& L);
hipError_t launch_gemm(const GemmLaunch& L, hipStream_t st);

// ---- other kernels ---------------------------------------------------------------------------
hipError_t launch_repack_q4_1(const uint8_t* canon, int n_out, int n_in, uint8_t* codes, uint8_t* sm, int G,
                              int col0, int gu_mode, hipStream_t st);
// gu: 0 plain run of tiles tile0.. (16 columns each); 1 / 2 the gate / up half of a gate|up image.
hipError_t launch_dequant_q4_1(const WMat& w, int tile0, int gu, int n_out, float* out, hipStream_t st);
hipError_t launch_rope_table(float2* table, int max_ctx, int hd, double base, hipStream_t st);
hipError_t launch_embed(const int32_t* tokens, int fill_token, int rows, const uint16_t* embed, int V, int H,
                        float scale, float* x, float* ss, hipStream_t st);
hipError_t launch_sumsq(const float* x, int ldx, int rows, int H, float* ss, hipStream_t st);
hipError_t launch_rmsnorm(const float* x, int ldx, int rows, int H, const uint16_t* g, float eps, uint16_t* out,
                          int ldo, hipStream_t st);

struct RopeAppend {
    const float* qkv = nullptr;  // [rows][ldq]: q | k | v
    int ldq = 0;
    int rows_q = 0;              // rows whose q heads are produced (the first rows_q rows)
    int rows = 0;                // rows whose k/v are appended (own plane)
    int split_row = 0;           // rows < split_row at pos0 + r, rows >= split_row at pos1 + (r - split_row)
    int pos0 = 0, pos1 = 0;
    int Hq = 0, nkv = 0, hd = 0;
    int own = 0;
    int qk_norm = 0;
    const uint16_t* q_norm = nullptr;
    const uint16_t* k_norm = nullptr;
    float eps = 0.f;
    const float2* rope = nullptr;  // [max_ctx][hd / 2] (cos, sin)
    void* plane = nullptr;         // own plane [max_ctx][2][w], fp32 or (kv_bf16) bf16 values
    int kv_bf16 = 0;
    int w = 0;
    float* q_out = nullptr;        // [rows_q][Hq][hd]
};
hipError_t launch_rope_append(const RopeAppend& a, hipStream_t st);

struct Attn {
    const float* qkv = nullptr;  // [rows][ldq] raw q | k | v of the layer's GEMM
    const float* ss = nullptr;   // [rows][ldq / 16] per-tile sums of squares (GEMM epilogue)
    int ldq = 0;
    const uint16_t* q_norm = nullptr;
    const uint16_t* k_norm = nullptr;
    int qk_norm = 0;
    float eps = 0.f;
    const float2* rope = nullptr;
    void* plane = nullptr;       // [max_ctx][2][w] (own or owner's), fp32 or (kv_bf16) bf16 values
    int kv_bf16 = 0;
    int ring_cap = 0;            // > 0: the plane is a ring of ring_cap slots, position p in slot p mod ring_cap
    int w = 0, own = 0;
    int M = 0, Hq = 0, nkv = 0, hd = 0;
    int causal = 1;              // 1: row m at pos0 + m sees [max(0, pos0 + m - window + 1), pos0 + m]
    int pos0 = 0;
    int window = 0;
    int ctx_lo = 0, ctx_hi = 0;  // draft: every row sees [ctx_lo, ctx_hi]
    // rows appended by this kernel (own layer): positions [np0, np1); row of p: p < sp ? r_lo + p - np0 : r_hi + p - sp
    int np0 = 0, np1 = 0, sp = 0, r_lo = 0, r_hi = 0;
    uint16_t* out = nullptr;     // [M][Hq * hd] bf16
    float* part = nullptr;       // scratch
    size_t part_floats = 0;
    int* counters = nullptr;     // zero between launches
    int n_counters = 0;
    int n_cu = 256;              // compute units of the device (chunk planning)
    // causal passes: the key chunks are planned for rows at pos_plan .. pos_plan + M - 1 (pos_plan >=
    // pos0), so passes at positions up to pos_plan share one launch configuration; 0: at pos0
    int pos_plan = 0;
    // passes replayed from a graph: the positions held P are read from *dpos at run time. Causal:
    // the rows sit at P .. P + M - 1. Draft block: the n_ctx context rows at P .., the block rows after
    // them, and window is the draft's context window. pos0, the new rows and the key range follow from P.
    const int64_t* dpos = nullptr;
    int n_ctx = 0;
};
size_t attn_part_floats_needed(const Attn& a);
// The launch configuration the attention takes for these arguments: chunks and sub-chunks per
// workgroup (the merge order of the partials follows from it).
int64_t attn_plan_key(const Attn& a);
hipError_t launch_set_i64(int64_t* dst, int64_t v, hipStream_t st);
hipError_t launch_attention(const Attn& a, hipStream_t st);

// Sampled draws instead of the argmax: 1/T (fp32), Philox key (seed) and counter offset words.
struct SampleArgs {
    float inv_t;
    uint32_t key0, key1, off0, off1;
};
hipError_t launch_argmax_accept(const float* logits, int k, int V, const int32_t* tokens, float* part_val,
                                int* part_idx, int nb, int32_t* out_tokens, int32_t* n_acc, int32_t* argmax_out,
                                hipStream_t st, const SampleArgs* sample = nullptr);
int argmax_blocks(int V);

// The allocation-free greedy accept keeps its argmax partials in a file-scope device array of the
// library (one per GPU): at most kMaxRows rows of at most kStaticAcceptBlocks spans of 4096 logits,
// i.e. a vocabulary of up to kStaticAcceptMaxVocab entries.
constexpr int kStaticAcceptBlocks = 256;
constexpr int kStaticAcceptMaxVocab = kStaticAcceptBlocks * 4096;
constexpr size_t kStaticAcceptScratchBytes = (size_t)kMaxRows * kStaticAcceptBlocks * 8;
// Device address of this device's array (hipGetSymbolAddress once per device, the device current).
hipError_t static_accept_scratch(int device, float** part_val, int** part_idx);
hipError_t launch_steer(float* logits, int k, int V, const int32_t* tok, const float* add, hipStream_t st);

}  // namespace bvf
