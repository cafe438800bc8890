// C ABI of the batched verify forward (include/bvf.h): descriptor checks, the device arena layout,
// weight loading (Q4_1 packed once at load, [PR2236] section 1), the per-layer KV-plane state
// ([PR2303] "What changes" item 1) and the launch sequence of a verify pass, the accept, and the
// DFlash draft block. Every entry point validates before it enqueues anything.
#include "bvf.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>
#include <vector>

#include "bvf_impl.hpp"

using namespace bvf;

namespace {

thread_local std::string g_err;

bvf_status fail(bvf_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

bvf_status ok() {
    g_err.clear();
    return BVF_OK;
}

#define HIP_TRY(expr)                                                                        \
    do {                                                                                     \
        hipError_t e_ = (expr);                                                              \
        if (e_ != hipSuccess) return fail(BVF_E_DEVICE, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

constexpr size_t kAlign = 256;
constexpr size_t kPartialFloats = (size_t)16 << 20;  // split-K scratch (64 MiB)
constexpr int kCounters = 16384;

struct Mat {
    WMat w;          // packed image (codes + sm), or bf16 matrix
    int n_out = 0;   // columns of the packed image (fused)
};

struct Layer {
    bvf_layer_desc d{};
    int w = 0;             // KV width (own or owner's)
    int qd = 0, kvd = 0;   // q width, own k/v width (0 on a shared layer)
    Mat qkv, o, gu, down;
    Mat ple_gate, ple_proj;   // per-layer embedding gate [ple_dim][H] and projection [H][ple_dim] (ple_dim > 0)
    uint16_t *attn_norm = nullptr, *mlp_norm = nullptr, *q_norm = nullptr, *k_norm = nullptr;
    uint16_t* layer_scalar = nullptr;   // one bf16 value (ple_dim > 0)
    void* plane = nullptr;    // own plane [cap][2][w] of fp32 or bf16 values (kv_bf16)
    int cap = 0;              // position slots of the own plane: max_ctx, or window + kRingSlack (ring)
    bool ring = false;        // position p lives in slot p mod cap
    const float2* rope = nullptr;
    unsigned loaded = 0;      // bit i: matrix i; bits 16..20: norms and the layer scalar
};
constexpr int kNormBit = 16;   // per-layer bf16 tensor bits start here (matrix ids take bits 0..8)
// Ring planes: the most rows one pass appends; a pass appending rows P..P+k-1 into a ring of
// window + kRingSlack slots overwrites only positions older than P - window + 1.
constexpr int kRingSlack = kMaxRows;

// Positions a plane holds at `held` positions: all of them, or on a ring the last `window`.
int64_t plane_keep(const Layer& L, int64_t held) { return L.ring ? std::min<int64_t>(held, L.d.window) : held; }

// Calls f(slot, first, count) for the runs of consecutive slots that positions [p0, p1) of a plane
// occupy (one run on a linear plane; up to two per pass round the ring); first = p - p0.
template <class F>
hipError_t for_slot_runs(const Layer& L, int64_t p0, int64_t p1, F f) {
    for (int64_t p = p0; p < p1;) {
        const int64_t slot = p % L.cap;
        const int64_t n = std::min<int64_t>(p1 - p, L.cap - slot);
        hipError_t e = f(slot, p - p0, n);
        if (e != hipSuccess) return e;
        p += n;
    }
    return hipSuccess;
}

// bf16 bits of fp32 values, rounded to nearest even (NaN kept quiet)
void round_to_bf16(const float* src, size_t n, std::vector<uint16_t>& out) {
    out.resize(n);
    for (size_t i = 0; i < n; ++i) {
        uint32_t u;
        std::memcpy(&u, &src[i], 4);
        out[i] = (u & 0x7fffffffu) > 0x7f800000u ? (uint16_t)((u >> 16) | 0x40u) : (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    }
}

}  // namespace

struct bvf_model {
    bvf_model_desc d{};
    std::vector<bvf_layer_desc> ld;
    std::vector<int32_t> taps;
    std::vector<Layer> L;
    hipStream_t st = nullptr;
    int device = 0;
    int n_cu = 256;          // compute units of the device (GEMM planning)
    uint8_t* arena = nullptr;
    size_t arena_bytes = 0;
    uint16_t *embed = nullptr, *final_norm = nullptr, *fc = nullptr, *hidden_norm = nullptr;
    uint16_t* ple_table = nullptr;   // [vocab][n_layers * ple_dim] (ple_dim > 0)
    uint16_t* pbuf = nullptr;        // [16][ple_dim] bf16 gated per-layer inputs (the projection's rows)
    unsigned loaded = 0;     // bit t: bf16 tensor t (model-wide)
    // scratch
    float* x = nullptr;
    uint16_t* act = nullptr;
    float* qkv = nullptr;
    float* qbuf = nullptr;
    uint16_t* obuf = nullptr;
    uint16_t* mbuf = nullptr;
    float* fcout = nullptr;
    float* partial = nullptr;
    int* counters = nullptr;
    float* attn_part = nullptr;
    size_t attn_part_floats = 0;
    float* ss_x = nullptr;     // [16][hidden / 16] per-tile sums of squares of the residual rows
    float* ss_qkv = nullptr;   // [16][nqkv_max / 16] per-tile sums of squares of q | k | v
    float* am_val = nullptr;
    int* am_idx = nullptr;
    int am_blocks = 0;
    float* logits_scratch = nullptr;
    float* logits_tmp = nullptr;     // verify model: head output of the GEMM timing entry
    uint8_t* staging = nullptr;
    size_t staging_bytes = 0;
    std::vector<std::pair<int, float2*>> rope_tables;
    int hd_max = 0, qd_max = 0, nqkv_max = 0, ffn_max = 0;
    int row_cap = kMaxRows;    // rows of the activation buffers: prefill chunks on verify models
    // state
    int64_t held = 0;
    int32_t pending = -1;
    // graph replay of the verify pass: captured on cap_st, launched on st; valid for one
    // (plan bound, k, tokens, logits, taps) key. The captured attention reads the positions held
    // from dpos, which a one-thread kernel sets before each replay.
    int use_graph = 0;
    hipStream_t cap_st = nullptr;
    hipGraphExec_t gexec = nullptr;
    int64_t* dpos = nullptr;
    int64_t g_plan = -1;
    int64_t n_captures = 0;
    int32_t g_k = 0;
    const void *g_tok = nullptr, *g_lg = nullptr, *g_taps = nullptr;
    // graph replays of the draft block: one capture per context-row count n_new, valid for one key
    // (the layers' attention plans, block, buffers, embedding scale, mask token, target model); the
    // captured attention reads the draft's positions held from dpos like the verify pass
    struct DraftGraph {
        hipGraphExec_t exec = nullptr;
        int64_t plan = -1;
        int32_t block = 0, mask = 0;
        float scale = 0.f;
        const void* ptr[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
    };
    DraftGraph dg[kMaxRows + 1];
    ~bvf_model() {
        if (gexec) (void)hipGraphExecDestroy(gexec);
        for (DraftGraph& g : dg)
            if (g.exec) (void)hipGraphExecDestroy(g.exec);
        if (cap_st) (void)hipStreamDestroy(cap_st);
    }
};

struct bvf_snapshot {
    int n_layers = 0;
    int64_t held = 0;
    int device = 0;
    int kv_elem = 4;   // bytes per stored K/V value
    std::vector<int64_t> per;
    std::vector<int> shared;
    std::vector<int> cap;        // position slots of each own plane (ring planes: window + 16)
    std::vector<int64_t> kept;   // positions kept of each own plane (ring planes: the last min(held, window))
    std::vector<int64_t> rows;   // rows allocated for each own plane (>= kept; bvf_snapshot_update reuses them)
    std::vector<float*> data;    // kept rows of each own plane, in position order
};

namespace {

bool is_draft(const bvf_model_desc& d) { return d.block_causal == 0; }

bvf_status check_desc(const bvf_model_desc* d) {
    if (!d) return fail(BVF_E_INVALID, "descriptor is NULL");
    if (d->n_layers < 1) return fail(BVF_E_INVALID, "n_layers %d < 1", d->n_layers);
    if (d->hidden < 128 || d->hidden % 128) return fail(BVF_E_INVALID, "hidden %d is not a positive multiple of 128", d->hidden);
    if (d->n_q_heads < 1) return fail(BVF_E_INVALID, "n_q_heads %d < 1", d->n_q_heads);
    if (d->max_ctx < 1 || d->max_ctx > (1 << 24)) return fail(BVF_E_INVALID, "max_ctx %d out of range", d->max_ctx);
    if (!d->layers) return fail(BVF_E_INVALID, "layers is NULL");
    if (d->block_causal != 0 && d->block_causal != 1) return fail(BVF_E_INVALID, "block_causal must be 0 or 1");
    if (d->rms_eps < 0.f || !(d->rope_base > 0.f)) return fail(BVF_E_INVALID, "rms_eps < 0 or rope_base <= 0");
    if (d->vocab < 0 || d->vocab % 16) return fail(BVF_E_INVALID, "vocab %d must be a non-negative multiple of 16", d->vocab);
    if (!is_draft(*d) && d->vocab < 16) return fail(BVF_E_INVALID, "a verify model needs vocab >= 16");
    if (d->n_taps < 0 || d->n_taps > 64) return fail(BVF_E_INVALID, "n_taps %d out of range", d->n_taps);
    if (d->n_taps > 0 && !d->tap_layers && !is_draft(*d)) return fail(BVF_E_INVALID, "tap_layers is NULL");
    if (is_draft(*d) && d->n_taps < 1) return fail(BVF_E_INVALID, "a draft needs n_taps >= 1 (fc input rows)");
    if (d->draft_window < 0) return fail(BVF_E_INVALID, "draft_window < 0");
    if (d->kv_bf16 != 0 && d->kv_bf16 != 1) return fail(BVF_E_INVALID, "kv_bf16 must be 0 or 1");
    if (d->ple_dim < 0 || d->ple_dim % 128 || d->ple_dim > 4096)
        return fail(BVF_E_INVALID, "ple_dim %d is not 0 or a multiple of 128 up to 4096", d->ple_dim);
    if (d->ple_dim > 0 && is_draft(*d)) return fail(BVF_E_INVALID, "per-layer embeddings exist on a verify model only");
    if (d->kv_ring != 0 && d->kv_ring != 1) return fail(BVF_E_INVALID, "kv_ring must be 0 or 1");
    if (d->kv_ring && is_draft(*d)) return fail(BVF_E_INVALID, "ring planes exist on a verify model only");
    if (!is_draft(*d))
        for (int t = 0; t < d->n_taps; ++t)
            if (d->tap_layers[t] < 0 || d->tap_layers[t] >= d->n_layers)
                return fail(BVF_E_INVALID, "tap layer %d does not fit a %d-layer model", d->tap_layers[t], d->n_layers);
    for (int l = 0; l < d->n_layers; ++l) {
        const bvf_layer_desc& L = d->layers[l];
        if (L.attn != BVF_ATTN_SLIDING && L.attn != BVF_ATTN_FULL) return fail(BVF_E_INVALID, "layer %d: attn %d", l, L.attn);
        if (L.head_dim != 64 && L.head_dim != 128 && L.head_dim != 256)
            return fail(BVF_E_INVALID, "layer %d: head_dim %d not in {64, 128, 256}", l, L.head_dim);
        if (L.n_kv_heads < 1 || d->n_q_heads % L.n_kv_heads)
            return fail(BVF_E_INVALID, "layer %d: n_kv_heads %d does not divide n_q_heads %d", l, L.n_kv_heads, d->n_q_heads);
        if ((d->n_q_heads * L.head_dim) % 128) return fail(BVF_E_INVALID, "layer %d: n_q_heads * head_dim not a multiple of 128", l);
        if (L.window < 0) return fail(BVF_E_INVALID, "layer %d: window < 0", l);
        if (L.ffn < 128 || L.ffn % 128) return fail(BVF_E_INVALID, "layer %d: ffn %d not a positive multiple of 128", l, L.ffn);
        if (L.kv_owner >= 0) {
            if (is_draft(*d)) return fail(BVF_E_INVALID, "layer %d: a draft layer cannot share KV", l);
            if (L.kv_owner >= l) return fail(BVF_E_INVALID, "layer %d: owner %d is not an earlier layer", l, L.kv_owner);
            const bvf_layer_desc& O = d->layers[L.kv_owner];
            if (O.kv_owner >= 0) return fail(BVF_E_INVALID, "layer %d: owner %d is itself shared", l, L.kv_owner);
            if (O.attn != L.attn || O.n_kv_heads != L.n_kv_heads || O.head_dim != L.head_dim)
                return fail(BVF_E_INVALID, "layer %d: owner %d has another attention type or geometry", l, L.kv_owner);
        } else if (L.kv_owner != -1) {
            return fail(BVF_E_INVALID, "layer %d: kv_owner %d", l, L.kv_owner);
        }
    }
    return BVF_OK;
}

// Lays the model out in the arena (base == nullptr: sizes only). Returns the bytes needed.
size_t layout(bvf_model* m, uint8_t* base) {
    size_t off = 0;
    auto take = [&](size_t bytes) -> uint8_t* {
        off = (off + kAlign - 1) / kAlign * kAlign;
        uint8_t* p = base ? base + off : nullptr;
        off += bytes;
        return p;
    };
    const bvf_model_desc& d = m->d;
    const int H = d.hidden;
    // verify models run prefill chunks of up to kMaxGemmRows rows through the same buffers
    const int RC = is_draft(d) ? kMaxRows : kMaxGemmRows;
    m->row_cap = RC;
    auto mat = [&](Mat& M, int n_out, int K) {
        M.n_out = n_out;
        M.w.n_tiles = n_out / kTile;
        M.w.G = K / kSuper;
        M.w.K = K;
        M.w.codes = take((size_t)M.w.n_tiles * M.w.G * 1024);
        M.w.sm = take((size_t)M.w.n_tiles * M.w.G * 256);
    };
    m->hd_max = m->qd_max = m->nqkv_max = m->ffn_max = 0;
    size_t staging = 0;
    m->L.assign(d.n_layers, Layer{});
    for (int l = 0; l < d.n_layers; ++l) {
        Layer& L = m->L[l];
        L.d = m->ld[l];
        const int hd = L.d.head_dim;
        L.qd = d.n_q_heads * hd;
        const bool own = L.d.kv_owner < 0;
        L.kvd = own ? L.d.n_kv_heads * hd : 0;
        L.w = m->ld[own ? l : L.d.kv_owner].n_kv_heads * m->ld[own ? l : L.d.kv_owner].head_dim;
        mat(L.qkv, L.qd + 2 * L.kvd, H);
        mat(L.o, H, L.qd);
        mat(L.gu, 2 * L.d.ffn, H);
        mat(L.down, H, L.d.ffn);
        if (d.ple_dim > 0) {
            mat(L.ple_gate, d.ple_dim, H);
            mat(L.ple_proj, H, d.ple_dim);
            L.layer_scalar = (uint16_t*)take(2);
        }
        L.attn_norm = (uint16_t*)take((size_t)H * 2);
        L.mlp_norm = (uint16_t*)take((size_t)H * 2);
        L.q_norm = (uint16_t*)take((size_t)hd * 2);
        L.k_norm = (uint16_t*)take((size_t)hd * 2);
        L.ring = own && d.kv_ring && L.d.attn == BVF_ATTN_SLIDING && L.d.window > 0 &&
                 L.d.window + kRingSlack < d.max_ctx;
        L.cap = L.ring ? L.d.window + kRingSlack : d.max_ctx;
        L.plane = own ? (void*)take((size_t)L.cap * 2 * L.w * (d.kv_bf16 ? 2 : 4)) : nullptr;
        m->hd_max = std::max(m->hd_max, hd);
        m->qd_max = std::max(m->qd_max, L.qd);
        m->nqkv_max = std::max(m->nqkv_max, L.qd + 2 * L.kvd);
        m->ffn_max = std::max(m->ffn_max, L.d.ffn);
        // largest canonical image one load call brings in (Q, K, V, O, GATE, UP, DOWN separately)
        for (size_t elems : {(size_t)L.qd * H, (size_t)L.kvd * H, (size_t)H * L.qd, (size_t)L.d.ffn * H,
                             (size_t)d.ple_dim * H})
            staging = std::max(staging, elems / 32 * 20);
    }
    m->embed = d.vocab > 0 && !is_draft(d) ? (uint16_t*)take((size_t)d.vocab * H * 2) : nullptr;
    m->final_norm = (uint16_t*)take((size_t)H * 2);
    m->ple_table = d.ple_dim > 0 ? (uint16_t*)take((size_t)d.vocab * d.n_layers * d.ple_dim * 2) : nullptr;
    m->pbuf = d.ple_dim > 0 ? (uint16_t*)take((size_t)RC * d.ple_dim * 2) : nullptr;
    if (is_draft(d)) {
        m->fc = (uint16_t*)take((size_t)H * d.n_taps * H * 2);
        m->hidden_norm = (uint16_t*)take((size_t)H * 2);
    }
    // RoPE tables, one per distinct head_dim
    m->rope_tables.clear();
    for (int l = 0; l < d.n_layers; ++l) {
        const int hd = m->L[l].d.head_dim;
        size_t i = 0;
        while (i < m->rope_tables.size() && m->rope_tables[i].first != hd) ++i;
        if (i == m->rope_tables.size())
            m->rope_tables.push_back({hd, (float2*)take((size_t)d.max_ctx * (hd / 2) * sizeof(float2))});
        m->L[l].rope = m->rope_tables[i].second;
    }
    m->x = (float*)take((size_t)RC * H * 4);
    m->act = (uint16_t*)take((size_t)RC * H * 2);
    m->qkv = (float*)take((size_t)RC * m->nqkv_max * 4);
    m->qbuf = (float*)take((size_t)RC * m->qd_max * 4);
    m->obuf = (uint16_t*)take((size_t)RC * m->qd_max * 2);
    m->mbuf = (uint16_t*)take((size_t)RC * m->ffn_max * 2);
    m->fcout = (float*)take((size_t)RC * H * 4);
    m->partial = (float*)take(kPartialFloats * 4);
    m->counters = (int*)take((size_t)kCounters * 4);
    m->dpos = (int64_t*)take(8);
    // attention partials: (query tiles x KV heads) <= (RC / 16) n_q_heads at RC rows, up to
    // kAttnMaxChunks chunks each
    m->attn_part_floats = (size_t)(RC / 16) * d.n_q_heads * kAttnMaxChunks * 16 * attn_part_ld(m->hd_max);
    m->attn_part = (float*)take(m->attn_part_floats * 4);
    m->ss_x = (float*)take((size_t)RC * (H / kTile) * 4);
    m->ss_qkv = (float*)take((size_t)RC * (m->nqkv_max / kTile) * 4);
    const int V = d.vocab;
    m->am_blocks = V > 0 ? argmax_blocks(V) : 1;
    m->am_val = (float*)take((size_t)kMaxRows * m->am_blocks * 4);
    m->am_idx = (int*)take((size_t)kMaxRows * m->am_blocks * 4);
    m->logits_scratch = is_draft(d) && V > 0 ? (float*)take((size_t)kMaxRows * V * 4) : nullptr;
    m->logits_tmp = !is_draft(d) ? (float*)take((size_t)kMaxRows * V * 4) : nullptr;
    m->staging_bytes = staging;
    m->staging = take(staging);
    return (off + kAlign - 1) / kAlign * kAlign;
}

void copy_desc(bvf_model* m, const bvf_model_desc* d) {
    m->d = *d;
    m->ld.assign(d->layers, d->layers + d->n_layers);
    m->taps.assign(d->tap_layers ? d->tap_layers : nullptr, d->tap_layers ? d->tap_layers + d->n_taps : nullptr);
    if (is_draft(*d)) m->taps.clear();
    m->d.layers = m->ld.data();
    m->d.tap_layers = m->taps.empty() ? nullptr : m->taps.data();
}

// Which part of which packed image a matrix id names.
struct Run {
    const Mat* mat;
    int tile0, stride, n_out, gu_mode, col0;
};

bvf_status matrix_run(const bvf_model* m, int layer, int matrix, Run& r) {
    if (layer < 0 || layer >= m->d.n_layers) return fail(BVF_E_INVALID, "layer %d out of range", layer);
    const Layer& L = m->L[layer];
    switch (matrix) {
        case BVF_Q: r = {&L.qkv, 0, 1, L.qd, 0, 0}; break;
        case BVF_K:
        case BVF_V:
            if (L.kvd == 0) return fail(BVF_E_INVALID, "layer %d is KV-shared: it has no K/V projection", layer);
            r = {&L.qkv, (L.qd + (matrix == BVF_V ? L.kvd : 0)) / kTile, 1, L.kvd, 0, L.qd + (matrix == BVF_V ? L.kvd : 0)};
            break;
        case BVF_O: r = {&L.o, 0, 1, m->d.hidden, 0, 0}; break;
        case BVF_GATE: r = {&L.gu, 0, 1, L.d.ffn, 1, 0}; break;
        case BVF_UP: r = {&L.gu, 0, 1, L.d.ffn, 2, 0}; break;
        case BVF_DOWN: r = {&L.down, 0, 1, m->d.hidden, 0, 0}; break;
        case BVF_PLE_GATE:
        case BVF_PLE_PROJ:
            if (m->d.ple_dim == 0) return fail(BVF_E_INVALID, "the model has no per-layer embeddings");
            r = matrix == BVF_PLE_GATE ? Run{&L.ple_gate, 0, 1, m->d.ple_dim, 0, 0} : Run{&L.ple_proj, 0, 1, m->d.hidden, 0, 0};
            break;
        default: return fail(BVF_E_INVALID, "matrix id %d", matrix);
    }
    return BVF_OK;
}

unsigned layer_needs(const bvf_model* m, int l) {
    const Layer& L = m->L[l];
    unsigned need = (1u << BVF_Q) | (1u << BVF_O) | (1u << BVF_GATE) | (1u << BVF_UP) | (1u << BVF_DOWN);
    if (L.kvd) need |= (1u << BVF_K) | (1u << BVF_V);
    need |= (1u << (kNormBit + 0)) | (1u << (kNormBit + 1));          // attn_norm, mlp_norm
    if (m->d.qk_norm) need |= (1u << (kNormBit + 2)) | (1u << (kNormBit + 3));
    if (m->d.ple_dim > 0) need |= (1u << BVF_PLE_GATE) | (1u << BVF_PLE_PROJ) | (1u << (kNormBit + 4));
    return need;
}

bvf_status check_loaded(const bvf_model* m) {
    for (int l = 0; l < m->d.n_layers; ++l) {
        const unsigned need = layer_needs(m, l);
        if ((m->L[l].loaded & need) != need) return fail(BVF_E_STATE, "layer %d: weights not all loaded", l);
    }
    unsigned need = 1u << BVF_FINAL_NORM;
    if (!is_draft(m->d)) need |= 1u << BVF_EMBED;
    else need |= (1u << BVF_FC) | (1u << BVF_HIDDEN_NORM);
    if (m->d.ple_dim > 0) need |= 1u << BVF_PLE_TABLE;
    if ((m->loaded & need) != need) return fail(BVF_E_STATE, "model-wide weights not all loaded");
    return BVF_OK;
}

GemmLaunch gemm_for(const bvf_model* m, const Mat& mat, int epi) {
    GemmLaunch g;
    g.w = mat.w;
    g.fmt = W_Q4_1;
    g.epi = epi;
    g.tile0 = 0;
    g.tile_stride = 1;
    g.n_run_tiles = mat.w.n_tiles;
    g.partial = m->partial;
    g.partial_floats = kPartialFloats;
    g.counters = m->counters;
    g.n_counters = kCounters;
    g.n_cu = m->n_cu;
    return g;
}

// Head: logits[r] = E . a[r] over the tied bf16 table [V][H]; a is either the bf16 rows A or, if
// xsrc is given, bf16(rmsnorm(xsrc rows) * gain) formed in the GEMM's staging (sums of squares of
// xsrc in the scratch owner's ss_x).
hipError_t launch_head(const bvf_model* target, const uint16_t* A, int rows, float* logits, hipStream_t st,
                       const bvf_model* scratch_owner, const float* xsrc = nullptr, const uint16_t* gain = nullptr,
                       int row0 = 0) {
    GemmLaunch g;
    g.w.codes = (const uint8_t*)target->embed;
    g.w.n_tiles = target->d.vocab / kTile;
    g.w.G = target->d.hidden / kSuper;
    g.w.K = target->d.hidden;
    g.fmt = W_BF16;
    g.epi = EPI_STORE;
    g.n_run_tiles = g.w.n_tiles;
    g.A = A;
    g.lda = target->d.hidden;
    g.M = rows;
    g.y = logits;
    g.ldy = target->d.vocab;
    g.partial = scratch_owner->partial;
    g.partial_floats = kPartialFloats;
    g.counters = scratch_owner->counters;
    g.n_counters = kCounters;
    g.n_cu = scratch_owner->n_cu;
    if (xsrc) {
        // rows row0 .. row0 + rows - 1 of xsrc and of the sums of squares
        g.xsrc = xsrc + (size_t)row0 * target->d.hidden; g.ldx = target->d.hidden; g.n_ss = target->d.hidden / kTile;
        g.ss_in = scratch_owner->ss_x + (size_t)row0 * g.n_ss;
        g.gain = gain; g.eps = scratch_owner->d.rms_eps;
    }
    return launch_gemm(g, st);
}

// Attention arguments of a layer (the fused norm/rope/append/attention kernel).
Attn attn_for(const bvf_model* m, const Layer& L, int rows) {
    Attn at;
    at.qkv = m->qkv; at.ss = m->ss_qkv; at.ldq = L.qkv.n_out;
    at.q_norm = L.q_norm; at.k_norm = L.k_norm; at.qk_norm = m->d.qk_norm; at.eps = m->d.rms_eps;
    at.rope = L.rope; at.w = L.w;
    at.M = rows; at.Hq = m->d.n_q_heads; at.nkv = L.d.n_kv_heads; at.hd = L.d.head_dim;
    at.out = m->obuf; at.part = m->attn_part; at.part_floats = m->attn_part_floats;
    at.n_cu = m->n_cu;
    at.counters = m->counters; at.n_counters = kCounters;
    return at;
}

// One verify layer over rows x [k][H] at positions P..P+k-1 (layer-major batched order, [PR2303]
// "What changes"): attention half, then the SwiGLU MLP half; an own layer appends its K/V rows, a
// KV-shared layer reads its owner's plane. The input rows' RMSNorms run inside the GEMMs' staging
// from the per-tile sums of squares in ss_x (written by the previous layer's down projection, or
// the embedding); the layer leaves ss_x for the next one. taps (optional): bf16 copy of the output.
// On a model with per-layer embeddings the layer ends with the PLE tail ([PR2303] "What changes":
// the PLE gate and projection as M-row GEMMs, then the layer scalar): the down projection leaves
// bf16(x) in act, the gate GEMM writes h = bf16(silu(Wg . act) * p) (p gathered by the rows'
// tokens), and the projection GEMM adds Wp . h to x and scales by the layer scalar.
// Causal passes plan their attention for a bound on the positions held: the last position of the
// 256-position span that holds P (at most max_ctx - k). Direct launches and graph replays at any P
// of one span then run the same chunk plan and agree bit for bit, and one captured pass serves the
// whole span.
constexpr int kPlanSpan = 256;
int plan_bound(const bvf_model* m, int64_t P, int k) {
    return (int)std::min<int64_t>(m->d.max_ctx - k, P | (kPlanSpan - 1));
}

// dpos (optional): the positions held are read from device memory at run time (captured passes).
hipError_t run_layer(bvf_model* m, int l, float* x, int k, int P, uint16_t* taps, int ldt, const int32_t* tokens,
                     const int64_t* dpos = nullptr) {
    Layer& L = m->L[l];
    const int H = m->d.hidden;
    hipStream_t st = m->st;
    hipError_t e;
    // Up to one 16-row tile the RMSNorms fold into the GEMMs' staging of fp32 x. Wider prefill chunks
    // run each norm once as its own kernel into bf16 rows instead: a 64-row chunk would otherwise have
    // every workgroup stage 64 fp32 rows (four times the bytes of the bf16 copy).
    GemmLaunch g = gemm_for(m, L.qkv, EPI_STORE);
    if (k > kMaxRows) {
        if ((e = launch_rmsnorm(x, H, k, H, L.attn_norm, m->d.rms_eps, m->act, H, st)) != hipSuccess) return e;
        g.A = m->act; g.lda = H;
    } else {
        g.xsrc = x; g.ldx = H; g.ss_in = m->ss_x; g.n_ss = H / kTile; g.gain = L.attn_norm; g.eps = m->d.rms_eps;
    }
    g.M = k; g.y = m->qkv; g.ldy = L.qkv.n_out; g.ss_out = m->ss_qkv;
    if ((e = launch_gemm(g, st)) != hipSuccess) return e;
    Attn at = attn_for(m, L, k);
    at.plane = L.plane ? L.plane : m->L[L.d.kv_owner].plane;
    {
        const Layer& src = L.plane ? L : m->L[L.d.kv_owner];
        at.ring_cap = src.ring ? src.cap : 0;
    }
    at.kv_bf16 = m->d.kv_bf16;
    at.own = L.plane != nullptr;
    at.causal = 1; at.pos0 = P; at.window = L.d.attn == BVF_ATTN_SLIDING ? L.d.window : 0;
    at.np0 = P; at.np1 = P + k; at.sp = P; at.r_lo = 0; at.r_hi = 0;
    at.pos_plan = plan_bound(m, P, k);
    at.dpos = dpos;
    if ((e = launch_attention(at, st)) != hipSuccess) return e;
    g = gemm_for(m, L.o, EPI_RESID);
    g.A = m->obuf; g.lda = L.qd; g.M = k; g.y = x; g.ldy = H; g.ss_out = m->ss_x;
    if ((e = launch_gemm(g, st)) != hipSuccess) return e;
    g = gemm_for(m, L.gu, EPI_SWIGLU);
    if (k > kMaxRows) {
        if ((e = launch_rmsnorm(x, H, k, H, L.mlp_norm, m->d.rms_eps, m->act, H, st)) != hipSuccess) return e;
        g.A = m->act; g.lda = H;
    } else {
        g.xsrc = x; g.ldx = H; g.ss_in = m->ss_x; g.n_ss = H / kTile; g.gain = L.mlp_norm; g.eps = m->d.rms_eps;
    }
    g.M = k; g.out = m->mbuf; g.ldo = L.d.ffn;
    if ((e = launch_gemm(g, st)) != hipSuccess) return e;
    g = gemm_for(m, L.down, EPI_RESID);
    g.A = m->mbuf; g.lda = L.d.ffn; g.M = k; g.y = x; g.ldy = H; g.ss_out = m->ss_x;
    g.taps = taps; g.ldt = ldt;
    if (m->d.ple_dim == 0) return launch_gemm(g, st);
    const int D = m->d.ple_dim;
    g.taps = m->act; g.ldt = H; g.ss_out = nullptr;
    if ((e = launch_gemm(g, st)) != hipSuccess) return e;
    g = gemm_for(m, L.ple_gate, EPI_PLE);
    g.A = m->act; g.lda = H; g.M = k; g.out = m->pbuf; g.ldo = D;
    g.tokens = tokens; g.ple = m->ple_table + (size_t)l * D; g.ple_ld = m->d.n_layers * D; g.vocab = m->d.vocab;
    if ((e = launch_gemm(g, st)) != hipSuccess) return e;
    g = gemm_for(m, L.ple_proj, EPI_RESID);
    g.A = m->pbuf; g.lda = D; g.M = k; g.y = x; g.ldy = H; g.ss_out = m->ss_x; g.rscale = L.layer_scalar;
    g.taps = taps; g.ldt = ldt;
    return launch_gemm(g, st);
}

}  // namespace

extern "C" {

const char* bvf_last_error(void) { return g_err.c_str(); }

int64_t bvf_cut_floats(const int64_t* per, int32_t n_per, int32_t plane, int64_t positions) {
    if (!per || n_per < 1 || plane < 0) return -1;
    return positions * 2 * per[plane < n_per ? plane : n_per - 1];
}

size_t bvf_arena_bytes(const bvf_model_desc* desc) {
    if (check_desc(desc) != BVF_OK) return 0;
    bvf_model tmp;
    copy_desc(&tmp, desc);
    const size_t n = layout(&tmp, nullptr);
    g_err.clear();
    return n;
}

bvf_status bvf_create(const bvf_model_desc* desc, void* d_arena, size_t arena_bytes, void* hip_stream, bvf_model** out) {
    if (!out) return fail(BVF_E_INVALID, "out is NULL");
    *out = nullptr;
    bvf_status s = check_desc(desc);
    if (s) return s;
    if (!d_arena) return fail(BVF_E_INVALID, "d_arena is NULL");
    if ((uintptr_t)d_arena % kAlign) return fail(BVF_E_INVALID, "d_arena is not 256-byte aligned");
    bvf_model* m = new bvf_model;
    copy_desc(m, desc);
    const size_t need = layout(m, nullptr);
    if (arena_bytes < need) {
        delete m;
        return fail(BVF_E_CAPACITY, "arena of %zu bytes < %zu needed", arena_bytes, need);
    }
    layout(m, (uint8_t*)d_arena);
    m->arena = (uint8_t*)d_arena;
    m->arena_bytes = arena_bytes;
    m->st = (hipStream_t)hip_stream;
    hipError_t e = hipGetDevice(&m->device);
    if (e == hipSuccess) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, m->device) == hipSuccess && n > 0) m->n_cu = n;
    }
    if (e == hipSuccess) e = hipMemsetAsync(d_arena, 0, need, m->st);
    for (auto& pr : m->rope_tables)
        if (e == hipSuccess) e = launch_rope_table(pr.second, m->d.max_ctx, pr.first, (double)m->d.rope_base, m->st);
    if (e == hipSuccess) e = hipStreamSynchronize(m->st);
    if (e != hipSuccess) {
        delete m;
        return fail(BVF_E_DEVICE, "create: %s", hipGetErrorString(e));
    }
    *out = m;
    return ok();
}

void bvf_destroy(bvf_model* m) { delete m; }

bvf_status bvf_load_q4_1(bvf_model* m, int32_t layer, int32_t matrix, const void* h_blocks, size_t bytes, int32_t n_out,
                         int32_t n_in) {
    if (!m) return fail(BVF_E_INVALID, "model is NULL");
    Run r;
    bvf_status s = matrix_run(m, layer, matrix, r);
    if (s) return s;
    if (n_out != r.n_out || n_in != r.mat->w.K)
        return fail(BVF_E_INVALID, "layer %d matrix %d: shape %d x %d, expected %d x %d", layer, matrix, n_out, n_in, r.n_out,
                    r.mat->w.K);
    const size_t need = (size_t)n_out * (n_in / 32) * 20;
    if (!h_blocks || bytes != need) return fail(BVF_E_INVALID, "Q4_1 image of %zu bytes, expected %zu", bytes, need);
    if (need > m->staging_bytes) return fail(BVF_E_CAPACITY, "staging too small");
    HIP_TRY(hipMemcpyAsync(m->staging, h_blocks, need, hipMemcpyHostToDevice, m->st));
    HIP_TRY(launch_repack_q4_1(m->staging, n_out, n_in, (uint8_t*)r.mat->w.codes, (uint8_t*)r.mat->w.sm, r.mat->w.G, r.col0,
                               r.gu_mode, m->st));
    HIP_TRY(hipStreamSynchronize(m->st));
    m->L[layer].loaded |= 1u << matrix;
    return ok();
}

bvf_status bvf_load_bf16(bvf_model* m, int32_t tensor, int32_t layer, const uint16_t* h, size_t n) {
    if (!m || !h) return fail(BVF_E_INVALID, "NULL argument");
    const int H = m->d.hidden;
    uint16_t* dst = nullptr;
    size_t want = 0;
    int bit = -1;
    auto per_layer = [&](int which) -> bvf_status {
        if (layer < 0 || layer >= m->d.n_layers) return fail(BVF_E_INVALID, "layer %d out of range", layer);
        Layer& L = m->L[layer];
        const int hd = L.d.head_dim;
        if (which == 4 && !L.layer_scalar) return fail(BVF_E_INVALID, "the model has no per-layer embeddings");
        uint16_t* ptrs[5] = {L.attn_norm, L.mlp_norm, L.q_norm, L.k_norm, L.layer_scalar};
        size_t sizes[5] = {(size_t)H, (size_t)H, (size_t)hd, (size_t)hd, 1};
        dst = ptrs[which];
        want = sizes[which];
        bit = kNormBit + which;
        return BVF_OK;
    };
    bvf_status s = BVF_OK;
    switch (tensor) {
        case BVF_EMBED:
            if (is_draft(m->d)) return fail(BVF_E_INVALID, "a draft uses the target's embedding table");
            dst = m->embed; want = (size_t)m->d.vocab * H; break;
        case BVF_FINAL_NORM: dst = m->final_norm; want = H; break;
        case BVF_ATTN_NORM: s = per_layer(0); break;
        case BVF_MLP_NORM: s = per_layer(1); break;
        case BVF_Q_NORM: s = per_layer(2); break;
        case BVF_K_NORM: s = per_layer(3); break;
        case BVF_FC:
            if (!is_draft(m->d)) return fail(BVF_E_INVALID, "fc exists on a draft only");
            dst = m->fc; want = (size_t)H * m->d.n_taps * H; break;
        case BVF_HIDDEN_NORM:
            if (!is_draft(m->d)) return fail(BVF_E_INVALID, "hidden norm exists on a draft only");
            dst = m->hidden_norm; want = H; break;
        case BVF_PLE_TABLE:
            if (m->d.ple_dim == 0) return fail(BVF_E_INVALID, "the model has no per-layer embeddings");
            dst = m->ple_table; want = (size_t)m->d.vocab * m->d.n_layers * m->d.ple_dim; break;
        case BVF_LAYER_SCALAR: s = per_layer(4); break;
        default: return fail(BVF_E_INVALID, "tensor id %d", tensor);
    }
    if (s) return s;
    if (n != want) return fail(BVF_E_INVALID, "tensor %d: %zu elements, expected %zu", tensor, n, want);
    HIP_TRY(hipMemcpyAsync(dst, h, n * 2, hipMemcpyHostToDevice, m->st));
    HIP_TRY(hipStreamSynchronize(m->st));
    if (bit >= 0) m->L[layer].loaded |= 1u << bit;
    else m->loaded |= 1u << tensor;
    return ok();
}

bvf_status bvf_set_kv(bvf_model* m, int32_t layer, const float* h_kv, int64_t positions) {
    if (!m || !h_kv) return fail(BVF_E_INVALID, "NULL argument");
    if (layer < 0 || layer >= m->d.n_layers) return fail(BVF_E_INVALID, "layer %d out of range", layer);
    Layer& L = m->L[layer];
    if (!L.plane) return fail(BVF_E_INVALID, "layer %d is KV-shared: it holds no plane", layer);
    if (positions < 0 || positions > m->d.max_ctx) return fail(BVF_E_CAPACITY, "positions %lld > max_ctx", (long long)positions);
    // a ring plane takes the last cap positions (older ones would be overwritten at once)
    const int64_t p0 = std::max<int64_t>(0, positions - L.cap);
    const size_t row = (size_t)2 * L.w, eb = m->d.kv_bf16 ? 2 : 4;
    std::vector<uint16_t> b;
    if (m->d.kv_bf16) round_to_bf16(h_kv + (size_t)p0 * row, (size_t)(positions - p0) * row, b);
    HIP_TRY(hipStreamSynchronize(m->st));
    HIP_TRY(for_slot_runs(L, p0, positions, [&](int64_t slot, int64_t first, int64_t n) {
        const void* src = m->d.kv_bf16 ? (const void*)(b.data() + (size_t)first * row) : (const void*)(h_kv + (size_t)(p0 + first) * row);
        return hipMemcpy((uint8_t*)L.plane + (size_t)slot * row * eb, src, (size_t)n * row * eb, hipMemcpyHostToDevice);
    }));
    return ok();
}

bvf_status bvf_get_kv(const bvf_model* m, int32_t layer, float* h_kv, int64_t positions) {
    if (!m || !h_kv) return fail(BVF_E_INVALID, "NULL argument");
    if (layer < 0 || layer >= m->d.n_layers) return fail(BVF_E_INVALID, "layer %d out of range", layer);
    const Layer& L = m->L[layer];
    if (!L.plane) return fail(BVF_E_INVALID, "layer %d is KV-shared: it holds no plane", layer);
    if (positions < 0 || positions > m->d.max_ctx) return fail(BVF_E_CAPACITY, "positions %lld > max_ctx", (long long)positions);
    const size_t row = (size_t)2 * L.w, eb = m->d.kv_bf16 ? 2 : 4;
    const int64_t p0 = positions - plane_keep(L, positions);   // older rows of a ring read as NaN
    const float qnan = std::numeric_limits<float>::quiet_NaN();
    std::fill(h_kv, h_kv + (size_t)p0 * row, qnan);
    std::vector<uint16_t> b(m->d.kv_bf16 ? (size_t)(positions - p0) * row : 0);
    HIP_TRY(hipStreamSynchronize(m->st));
    HIP_TRY(for_slot_runs(L, p0, positions, [&](int64_t slot, int64_t first, int64_t n) {
        void* dst = m->d.kv_bf16 ? (void*)(b.data() + (size_t)first * row) : (void*)(h_kv + (size_t)(p0 + first) * row);
        return hipMemcpy(dst, (const uint8_t*)L.plane + (size_t)slot * row * eb, (size_t)n * row * eb, hipMemcpyDeviceToHost);
    }));
    for (size_t i = 0; i < b.size(); ++i) {
        const uint32_t u = (uint32_t)b[i] << 16;
        std::memcpy(&h_kv[(size_t)p0 * row + i], &u, 4);
    }
    return ok();
}

bvf_status bvf_set_positions(bvf_model* m, int64_t positions) {
    if (!m) return fail(BVF_E_INVALID, "model is NULL");
    if (positions < 0 || positions > m->d.max_ctx) return fail(BVF_E_CAPACITY, "positions %lld out of [0, max_ctx]", (long long)positions);
    m->held = positions;
    m->pending = -1;
    return ok();
}

bvf_status bvf_kv_widths(const bvf_model* m, int64_t* out, int32_t n) {
    if (!m || !out || n != m->d.n_layers) return fail(BVF_E_INVALID, "need an array of n_layers entries");
    for (int l = 0; l < n; ++l) out[l] = m->L[l].w;
    return ok();
}

bvf_status bvf_plane_floats(const bvf_model* m, int64_t* out, int32_t n) {
    if (!m || !out || n != m->d.n_layers) return fail(BVF_E_INVALID, "need an array of n_layers entries");
    for (int l = 0; l < n; ++l) out[l] = m->L[l].plane ? plane_keep(m->L[l], m->held) * 2 * m->L[l].w : 0;
    return ok();
}

bvf_status bvf_positions_held(const bvf_model* m, int64_t* out) {
    if (!m || !out) return fail(BVF_E_INVALID, "NULL argument");
    *out = m->held;
    return ok();
}

}  // extern "C"

namespace {
// The verify pass's launches on stream st (positions P .. P + k - 1; with dpos, P read from there).
hipError_t enqueue_verify(bvf_model* m, hipStream_t st, const int32_t* d_tokens, int k, float* d_logits_all,
                          uint16_t* d_taps, const int64_t* dpos) {
    const int H = m->d.hidden, V = m->d.vocab, P = (int)m->held;
    const int T = (int)m->taps.size();
    hipStream_t saved = m->st;
    m->st = st;
    hipError_t e = launch_embed(d_tokens, -1, k, m->embed, V, H, 1.0f, m->x, m->ss_x, st);
    for (int l = 0; l < m->d.n_layers && e == hipSuccess; ++l) {
        uint16_t* taps_l = nullptr;
        if (d_taps)
            for (int t = 0; t < T; ++t)
                if (m->taps[t] == l) taps_l = d_taps + (size_t)t * H;
        e = run_layer(m, l, m->x, k, P, taps_l, T * H, d_tokens, dpos);
    }
    if (e == hipSuccess) e = launch_head(m, nullptr, k, d_logits_all, st, m, m->x, m->final_norm);
    m->st = saved;
    return e;
}

// The draft's context rows from their taps: fc ([CARD] "Draft": the tapped target features
// projected to the hidden size), then RMSNorm with the hidden-norm gain, into the rows of the A
// buffer that follow the B block rows.
hipError_t enqueue_draft_fc(bvf_model* dr, const uint16_t* d_new_taps, int n_new, int B, hipStream_t st) {
    if (n_new == 0) return hipSuccess;
    const int H = dr->d.hidden, T = dr->d.n_taps;
    GemmLaunch g;
    g.w.codes = (const uint8_t*)dr->fc;
    g.w.n_tiles = H / kTile;
    g.w.G = T * H / kSuper;
    g.w.K = T * H;
    g.fmt = W_BF16;
    g.epi = EPI_STORE;
    g.n_run_tiles = g.w.n_tiles;
    g.A = d_new_taps; g.lda = T * H; g.M = n_new; g.y = dr->fcout; g.ldy = H;
    g.partial = dr->partial; g.partial_floats = kPartialFloats; g.counters = dr->counters; g.n_counters = kCounters;
    g.n_cu = dr->n_cu;
    hipError_t e = launch_gemm(g, st);
    if (e != hipSuccess) return e;
    return launch_rmsnorm(dr->fcout, H, n_new, H, dr->hidden_norm, dr->d.rms_eps, dr->act + (size_t)B * H, H, st);
}

// Attention arguments of draft layer l for a block of B rows after n_new context rows ([CARD]
// "Draft"; [PR2236] section 2): the block rows 0..B-1 sit at s .. s + B - 1 and the context rows
// B.. at s_old .. s - 1 (s = s_old + n_new, s_old = the draft's positions held); both are appended,
// and the block sees the last draft_window context positions and every block row. With dpos the
// positions held are read from device memory (graph replays).
Attn draft_attn(bvf_model* dr, int l, int n_new, int B, const int64_t* dpos) {
    Layer& L = dr->L[l];
    const int s_old = (int)dr->held, s_new = s_old + n_new;
    Attn at = attn_for(dr, L, B);
    at.plane = L.plane; at.kv_bf16 = dr->d.kv_bf16; at.own = 1;
    at.causal = 0; at.pos0 = s_new;
    at.ctx_lo = (dr->d.draft_window > 0 && s_new - dr->d.draft_window > 0) ? s_new - dr->d.draft_window : 0;
    at.ctx_hi = s_new + B - 1;
    at.np0 = s_old; at.np1 = s_new + B; at.sp = s_new; at.r_lo = B; at.r_hi = 0;
    at.window = dr->d.draft_window; at.n_ctx = n_new; at.dpos = dpos;
    return at;
}

// The draft block's launches on stream st: the context rows (fc), the block rows [last token,
// mask x (B - 1)] through the draft layers, the final norm and the target's head on rows 1..B-1,
// their argmax. Every RMSNorm of the block rows is folded into the staging of the GEMM that reads
// them, from the per-tile sums of squares that the embedding and the o and down GEMMs leave in ss_x:
// the attention norm into q|k|v (whose rows B.. are the context rows, copied as fc's hidden norm
// left them), the MLP norm into gate|up, the final norm into the head.
hipError_t enqueue_draft(bvf_model* dr, const bvf_model* tg, const uint16_t* d_new_taps, int n_new,
                         const int32_t* d_last_token, int B, float embedding_scale, int mask_token, int32_t* d_proposals,
                         float* d_logits, hipStream_t st, const int64_t* dpos) {
    const int H = dr->d.hidden, V = tg->d.vocab;
    hipError_t e = enqueue_draft_fc(dr, d_new_taps, n_new, B, st);
    if (e != hipSuccess) return e;
    if ((e = launch_embed(d_last_token, mask_token, B, tg->embed, V, H, embedding_scale, dr->x, dr->ss_x, st)) != hipSuccess)
        return e;
    for (int l = 0; l < dr->d.n_layers; ++l) {
        Layer& L = dr->L[l];
        GemmLaunch g = gemm_for(dr, L.qkv, EPI_STORE);
        g.xsrc = dr->x; g.ldx = H; g.ss_in = dr->ss_x; g.n_ss = H / kTile; g.gain = L.attn_norm; g.eps = dr->d.rms_eps;
        g.n_fold = B;
        g.A = dr->act; g.lda = H; g.M = B + n_new; g.y = dr->qkv; g.ldy = L.qkv.n_out; g.ss_out = dr->ss_qkv;
        if ((e = launch_gemm(g, st)) != hipSuccess) return e;
        if ((e = launch_attention(draft_attn(dr, l, n_new, B, dpos), st)) != hipSuccess) return e;
        g = gemm_for(dr, L.o, EPI_RESID);
        g.A = dr->obuf; g.lda = L.qd; g.M = B; g.y = dr->x; g.ldy = H; g.ss_out = dr->ss_x;
        if ((e = launch_gemm(g, st)) != hipSuccess) return e;
        g = gemm_for(dr, L.gu, EPI_SWIGLU);
        g.xsrc = dr->x; g.ldx = H; g.ss_in = dr->ss_x; g.n_ss = H / kTile; g.gain = L.mlp_norm; g.eps = dr->d.rms_eps;
        g.M = B; g.out = dr->mbuf; g.ldo = L.d.ffn;
        if ((e = launch_gemm(g, st)) != hipSuccess) return e;
        g = gemm_for(dr, L.down, EPI_RESID);
        g.A = dr->mbuf; g.lda = L.d.ffn; g.M = B; g.y = dr->x; g.ldy = H; g.ss_out = dr->ss_x;
        if ((e = launch_gemm(g, st)) != hipSuccess) return e;
    }
    float* logits = d_logits ? d_logits : dr->logits_scratch;
    if ((e = launch_head(tg, nullptr, B - 1, logits, st, dr, dr->x, dr->final_norm, 1)) != hipSuccess) return e;
    return launch_argmax_accept(logits, B - 1, V, nullptr, dr->am_val, dr->am_idx, argmax_blocks(V), nullptr, nullptr,
                                d_proposals, st);
}
}  // namespace

extern "C" {

bvf_status bvf_verify_batch(bvf_model* m, const int32_t* d_tokens, int32_t k, float* d_logits_all, uint16_t* d_taps) {
    if (!m || !d_tokens || !d_logits_all) return fail(BVF_E_INVALID, "NULL argument");
    if (is_draft(m->d)) return fail(BVF_E_INVALID, "verify on a draft model");
    if (k < 1 || k > kMaxRows) return fail(BVF_E_INVALID, "k = %d outside [1, %d]", k, kMaxRows);
    if (m->held + k > m->d.max_ctx)
        return fail(BVF_E_CAPACITY, "%lld held + %d rows > max_ctx %d", (long long)m->held, k, m->d.max_ctx);
    bvf_status s = check_loaded(m);
    if (s) return s;
    if (!m->use_graph) {
        HIP_TRY(enqueue_verify(m, m->st, d_tokens, k, d_logits_all, d_taps, nullptr));
    } else {
        const int64_t plan = plan_bound(m, m->held, k);
        if (!m->gexec || m->g_plan != plan || m->g_k != k || m->g_tok != d_tokens || m->g_lg != d_logits_all ||
            m->g_taps != d_taps) {
            if (m->gexec) {
                HIP_TRY(hipGraphExecDestroy(m->gexec));
                m->gexec = nullptr;
            }
            if (!m->cap_st) HIP_TRY(hipStreamCreateWithFlags(&m->cap_st, hipStreamNonBlocking));
            hipGraph_t graph = nullptr;
            HIP_TRY(hipStreamBeginCapture(m->cap_st, hipStreamCaptureModeThreadLocal));
            hipError_t e = enqueue_verify(m, m->cap_st, d_tokens, k, d_logits_all, d_taps, m->dpos);
            hipError_t e2 = hipStreamEndCapture(m->cap_st, &graph);
            if (e != hipSuccess || e2 != hipSuccess) {
                if (graph) (void)hipGraphDestroy(graph);
                return fail(BVF_E_DEVICE, "graph capture: %s", hipGetErrorString(e != hipSuccess ? e : e2));
            }
            e = hipGraphInstantiate(&m->gexec, graph, nullptr, nullptr, 0);
            (void)hipGraphDestroy(graph);
            if (e != hipSuccess) {
                m->gexec = nullptr;
                return fail(BVF_E_DEVICE, "graph instantiate: %s", hipGetErrorString(e));
            }
            m->g_plan = plan; m->g_k = k;
            ++m->n_captures; m->g_tok = d_tokens; m->g_lg = d_logits_all; m->g_taps = d_taps;
        }
        HIP_TRY(launch_set_i64(m->dpos, m->held, m->st));
        HIP_TRY(hipGraphLaunch(m->gexec, m->st));
    }
    m->held += k;
    m->pending = k;
    return ok();
}

bvf_status bvf_prefill(bvf_model* m, const int32_t* d_tokens, int32_t n, float* d_last_logits) {
    if (!m || !d_tokens) return fail(BVF_E_INVALID, "NULL argument");
    if (is_draft(m->d)) return fail(BVF_E_INVALID, "prefill on a draft model");
    if (n < 1) return fail(BVF_E_INVALID, "n = %d < 1", n);
    if (m->pending >= 0) return fail(BVF_E_STATE, "a verify of %d rows is pending: commit it first", m->pending);
    if (m->held + n > m->d.max_ctx)
        return fail(BVF_E_CAPACITY, "%lld held + %d rows > max_ctx %d", (long long)m->held, n, m->d.max_ctx);
    bvf_status s = check_loaded(m);
    if (s) return s;
    const int H = m->d.hidden, V = m->d.vocab;
    for (int off = 0; off < n; off += m->row_cap) {
        const int c = std::min(m->row_cap, n - off);
        const int P = (int)m->held;
        HIP_TRY(launch_embed(d_tokens + off, -1, c, m->embed, V, H, 1.0f, m->x, m->ss_x, m->st));
        for (int l = 0; l < m->d.n_layers; ++l) HIP_TRY(run_layer(m, l, m->x, c, P, nullptr, 0, d_tokens + off));
        m->held += c;
        // the head on the last row of the last chunk only
        if (off + c == n && d_last_logits) HIP_TRY(launch_head(m, nullptr, 1, d_last_logits, m->st, m, m->x, m->final_norm, c - 1));
    }
    return ok();
}

bvf_status bvf_set_graph_mode(bvf_model* m, int32_t on) {
    if (!m) return fail(BVF_E_INVALID, "model is NULL");
    if (on != 0 && on != 1) return fail(BVF_E_INVALID, "graph mode must be 0 or 1");
    m->use_graph = on;
    return ok();
}

bvf_status bvf_graph_captures(const bvf_model* m, int64_t* out) {
    if (!m || !out) return fail(BVF_E_INVALID, "NULL argument");
    *out = m->n_captures;
    return ok();
}

bvf_status bvf_accept_greedy(bvf_model* m, const float* d_logits_all, int32_t k, const int32_t* d_tokens,
                             int32_t* d_out_tokens, int32_t* d_n_accepted) {
    if (!m || !d_logits_all || !d_tokens || !d_out_tokens || !d_n_accepted) return fail(BVF_E_INVALID, "NULL argument");
    if (is_draft(m->d)) return fail(BVF_E_INVALID, "accept on a draft model");
    if (k < 1 || k > kMaxRows) return fail(BVF_E_INVALID, "k = %d outside [1, %d]", k, kMaxRows);
    HIP_TRY(launch_argmax_accept(d_logits_all, k, m->d.vocab, d_tokens, m->am_val, m->am_idx, m->am_blocks, d_out_tokens,
                                 d_n_accepted, nullptr, m->st));
    return ok();
}

bvf_status bvf_accept_greedy_static(const float* d_logits_all, int32_t k, int32_t vocab, const int32_t* d_tokens,
                                    int32_t* d_out_tokens, int32_t* d_n_accepted, void* hip_stream) {
    if (!d_logits_all || !d_tokens || !d_out_tokens || !d_n_accepted) return fail(BVF_E_INVALID, "NULL argument");
    if (k < 1 || k > kMaxRows) return fail(BVF_E_INVALID, "k = %d outside [1, %d]", k, kMaxRows);
    if (vocab < 1 || vocab > kStaticAcceptMaxVocab)
        return fail(BVF_E_CAPACITY, "vocab %d outside [1, %d] (the static scratch holds %d spans of 4096 per row)", vocab,
                    kStaticAcceptMaxVocab, kStaticAcceptBlocks);
    int device = -1;
    HIP_TRY(hipGetDevice(&device));
    float* pv = nullptr;
    int* pi = nullptr;
    HIP_TRY(static_accept_scratch(device, &pv, &pi));
    HIP_TRY(launch_argmax_accept(d_logits_all, k, vocab, d_tokens, pv, pi, argmax_blocks(vocab), d_out_tokens,
                                 d_n_accepted, nullptr, (hipStream_t)hip_stream));
    return ok();
}

bvf_status bvf_accept_sampled(bvf_model* m, const float* d_logits_all, int32_t k, const int32_t* d_tokens, float temperature,
                              uint64_t seed, uint64_t offset, int32_t* d_out_tokens, int32_t* d_n_accepted,
                              int32_t* d_draws) {
    if (!m || !d_logits_all || !d_tokens || !d_out_tokens || !d_n_accepted) return fail(BVF_E_INVALID, "NULL argument");
    if (is_draft(m->d)) return fail(BVF_E_INVALID, "accept on a draft model");
    if (k < 1 || k > kMaxRows) return fail(BVF_E_INVALID, "k = %d outside [1, %d]", k, kMaxRows);
    if (!(temperature > 0.f) || !std::isfinite(temperature))
        return fail(BVF_E_INVALID, "temperature must be finite and > 0 (the greedy accept covers T = 0)");
    SampleArgs sa;
    sa.inv_t = 1.0f / temperature;
    sa.key0 = (uint32_t)seed;
    sa.key1 = (uint32_t)(seed >> 32);
    sa.off0 = (uint32_t)offset;
    sa.off1 = (uint32_t)(offset >> 32);
    HIP_TRY(launch_argmax_accept(d_logits_all, k, m->d.vocab, d_tokens, m->am_val, m->am_idx, m->am_blocks, d_out_tokens,
                                 d_n_accepted, d_draws, m->st, &sa));
    return ok();
}

bvf_status bvf_steer_logits(bvf_model* m, float* d_logits_all, int32_t k, const int32_t* d_tok, const float* d_add) {
    if (!m || !d_logits_all || !d_tok || !d_add) return fail(BVF_E_INVALID, "NULL argument");
    if (k < 1 || k > kMaxRows) return fail(BVF_E_INVALID, "k = %d outside [1, %d]", k, kMaxRows);
    HIP_TRY(launch_steer(d_logits_all, k, m->d.vocab, d_tok, d_add, m->st));
    return ok();
}

bvf_status bvf_extend_context(bvf_model* m, const float* h_kv_all, int64_t n) {
    if (!m) return fail(BVF_E_INVALID, "model is NULL");
    if (n < 0) return fail(BVF_E_INVALID, "n = %lld < 0", (long long)n);
    if (n > 0 && !h_kv_all) return fail(BVF_E_INVALID, "NULL argument");
    if (m->pending >= 0) return fail(BVF_E_STATE, "extend_context while a verify of %d rows is pending", m->pending);
    if (m->held + n > m->d.max_ctx)
        return fail(BVF_E_CAPACITY, "%lld held + %lld rows > max_ctx %d", (long long)m->held, (long long)n, m->d.max_ctx);
    if (n == 0) return ok();
    // every own plane takes its n rows at its own width, after the held positions (the rows of the
    // own layers follow one another in layer order in h_kv_all)
    HIP_TRY(hipStreamSynchronize(m->st));
    size_t off = 0;
    std::vector<uint16_t> b;
    for (int l = 0; l < m->d.n_layers; ++l) {
        Layer& L = m->L[l];
        if (!L.plane) continue;
        const size_t row = (size_t)2 * L.w, eb = m->d.kv_bf16 ? 2 : 4;
        // positions held .. held + n - 1 go to their slots; on a ring only the last cap of them stay
        const int64_t q0 = m->held + std::max<int64_t>(0, n - L.cap), q1 = m->held + n;
        const float* src = h_kv_all + off + (size_t)(q0 - m->held) * row;
        if (m->d.kv_bf16) round_to_bf16(src, (size_t)(q1 - q0) * row, b);   // bf16 planes: RNE, NaN kept quiet
        HIP_TRY(for_slot_runs(L, q0, q1, [&](int64_t slot, int64_t first, int64_t cnt) {
            const void* from = m->d.kv_bf16 ? (const void*)(b.data() + (size_t)first * row) : (const void*)(src + (size_t)first * row);
            return hipMemcpy((uint8_t*)L.plane + (size_t)slot * row * eb, from, (size_t)cnt * row * eb, hipMemcpyHostToDevice);
        }));
        off += (size_t)n * row;
    }
    m->held += n;
    return ok();
}

bvf_status bvf_commit_verify_rows(bvf_model* m, int32_t n) {
    if (!m) return fail(BVF_E_INVALID, "model is NULL");
    if (m->pending < 0) return fail(BVF_E_STATE, "commit_verify_rows with no verify pending");
    if (n < 0 || n > m->pending) return fail(BVF_E_STATE, "commit_verify_rows(%d) after a verify of %d rows", n, m->pending);
    m->held = m->held - m->pending + n;
    m->pending = -1;
    return ok();
}

bvf_status bvf_snapshot_take(bvf_model* m, bvf_snapshot** out) {
    if (!m || !out) return fail(BVF_E_INVALID, "NULL argument");
    *out = nullptr;
    if (m->pending >= 0)
        return fail(BVF_E_STATE, "snapshot while a verify of %d rows is pending: commit it first", m->pending);
    bvf_snapshot* s = new bvf_snapshot;
    s->n_layers = m->d.n_layers;
    s->held = m->held;
    s->device = m->device;
    s->kv_elem = m->d.kv_bf16 ? 2 : 4;
    for (int l = 0; l < m->d.n_layers; ++l) {
        const Layer& L = m->L[l];
        s->per.push_back(L.w);
        s->shared.push_back(L.plane ? 0 : 1);
        s->cap.push_back(L.plane ? L.cap : 0);
        s->kept.push_back(L.plane ? plane_keep(L, m->held) : 0);
        s->rows.push_back(s->kept.back());
        s->data.push_back(nullptr);
    }
    for (int l = 0; l < m->d.n_layers; ++l) {
        if (s->shared[l] || s->kept[l] == 0) continue;
        const Layer& L = m->L[l];
        const size_t row = (size_t)2 * L.w * s->kv_elem;
        hipError_t e = hipMalloc((void**)&s->data[l], (size_t)s->kept[l] * row);
        if (e == hipSuccess)
            e = for_slot_runs(L, s->held - s->kept[l], s->held, [&](int64_t slot, int64_t first, int64_t n) {
                return hipMemcpyAsync((uint8_t*)s->data[l] + (size_t)first * row, (const uint8_t*)L.plane + (size_t)slot * row,
                                      (size_t)n * row, hipMemcpyDeviceToDevice, m->st);
            });
        if (e != hipSuccess) {
            bvf_snapshot_free(s);
            return fail(BVF_E_DEVICE, "snapshot: %s", hipGetErrorString(e));
        }
    }
    hipError_t e = hipStreamSynchronize(m->st);
    if (e != hipSuccess) {
        bvf_snapshot_free(s);
        return fail(BVF_E_DEVICE, "snapshot: %s", hipGetErrorString(e));
    }
    *out = s;
    return ok();
}

namespace {
// A snapshot fits a model when the layer count, the widths, own/shared, the plane capacities and the
// stored element size agree.
bvf_status snapshot_fits(const bvf_model* m, const bvf_snapshot* s) {
    if (s->n_layers != m->d.n_layers)
        return fail(BVF_E_INVALID, "snapshot of %d layers, model of %d", s->n_layers, m->d.n_layers);
    for (int l = 0; l < m->d.n_layers; ++l) {
        if (s->per[l] != m->L[l].w) return fail(BVF_E_INVALID, "layer %d: snapshot width %lld, model %d", l, (long long)s->per[l], m->L[l].w);
        if (s->shared[l] != (m->L[l].plane ? 0 : 1)) return fail(BVF_E_INVALID, "layer %d: shared/own mismatch", l);
        if (s->cap[l] != (m->L[l].plane ? m->L[l].cap : 0))
            return fail(BVF_E_INVALID, "layer %d: snapshot plane of %d positions, model plane of %d (ring and linear planes differ)",
                        l, s->cap[l], m->L[l].plane ? m->L[l].cap : 0);
    }
    if (s->kv_elem != (m->d.kv_bf16 ? 2 : 4)) return fail(BVF_E_INVALID, "snapshot of %s planes, model of %s planes",
                                                           s->kv_elem == 2 ? "bf16" : "fp32", m->d.kv_bf16 ? "bf16" : "fp32");
    return BVF_OK;
}
}  // namespace

bvf_status bvf_snapshot_update(bvf_model* m, bvf_snapshot* s) {
    if (!m || !s) return fail(BVF_E_INVALID, "NULL argument");
    if (m->pending >= 0)
        return fail(BVF_E_STATE, "snapshot while a verify of %d rows is pending: commit it first", m->pending);
    bvf_status st = snapshot_fits(m, s);
    if (st) return st;
    std::vector<int64_t> kept(m->d.n_layers, 0);
    for (int l = 0; l < m->d.n_layers; ++l) {
        if (!m->L[l].plane) continue;
        kept[l] = plane_keep(m->L[l], m->held);
        if (kept[l] > s->rows[l])
            return fail(BVF_E_CAPACITY, "layer %d: %lld positions to keep, the snapshot holds room for %lld", l,
                        (long long)kept[l], (long long)s->rows[l]);
    }
    for (int l = 0; l < m->d.n_layers; ++l) {
        if (kept[l] == 0) continue;
        const Layer& L = m->L[l];
        const size_t row = (size_t)2 * L.w * s->kv_elem;
        HIP_TRY(for_slot_runs(L, m->held - kept[l], m->held, [&](int64_t slot, int64_t first, int64_t n) {
            return hipMemcpyAsync((uint8_t*)s->data[l] + (size_t)first * row, (const uint8_t*)L.plane + (size_t)slot * row,
                                  (size_t)n * row, hipMemcpyDeviceToDevice, m->st);
        }));
    }
    HIP_TRY(hipStreamSynchronize(m->st));
    s->held = m->held;
    s->kept = kept;
    return ok();
}

bvf_status bvf_restore(bvf_model* m, const bvf_snapshot* s) {
    if (!m || !s) return fail(BVF_E_INVALID, "NULL argument");
    bvf_status st = snapshot_fits(m, s);
    if (st) return st;
    if (s->held > m->d.max_ctx) return fail(BVF_E_CAPACITY, "snapshot holds more positions than max_ctx");
    for (int l = 0; l < m->d.n_layers; ++l) {
        if (s->shared[l] || !s->data[l] || s->kept[l] == 0) continue;
        const Layer& L = m->L[l];
        const size_t row = (size_t)2 * L.w * s->kv_elem;
        HIP_TRY(for_slot_runs(L, s->held - s->kept[l], s->held, [&](int64_t slot, int64_t first, int64_t n) {
            return hipMemcpyAsync((uint8_t*)L.plane + (size_t)slot * row, (const uint8_t*)s->data[l] + (size_t)first * row,
                                  (size_t)n * row, hipMemcpyDeviceToDevice, m->st);
        }));
    }
    HIP_TRY(hipStreamSynchronize(m->st));
    m->held = s->held;
    m->pending = -1;
    return ok();
}

bvf_status bvf_snapshot_floats(const bvf_snapshot* s, int64_t* out, int32_t n) {
    if (!s || !out || n != s->n_layers) return fail(BVF_E_INVALID, "need an array of n_layers entries");
    for (int l = 0; l < n; ++l) out[l] = s->shared[l] ? 0 : bvf_cut_floats(s->per.data(), s->n_layers, l, s->kept[l]);
    return ok();
}

void bvf_snapshot_free(bvf_snapshot* s) {
    if (!s) return;
    for (float* p : s->data)
        if (p) (void)hipFree(p);
    delete s;
}

bvf_status bvf_draft_block_forward(bvf_model* dr, const bvf_model* tg, const uint16_t* d_new_taps, int32_t n_new,
                                   const int32_t* d_last_token, int32_t block, float embedding_scale, int32_t mask_token,
                                   int32_t* d_proposals, float* d_logits) {
    if (!dr || !tg) return fail(BVF_E_INVALID, "NULL argument");
    if (block != 0 && (!d_last_token || !d_proposals)) return fail(BVF_E_INVALID, "NULL argument");
    if (!is_draft(dr->d)) return fail(BVF_E_INVALID, "the first model is not a draft");
    if (is_draft(tg->d)) return fail(BVF_E_INVALID, "the second model is not a verify (target) model");
    if (tg->d.hidden != dr->d.hidden) return fail(BVF_E_INVALID, "draft hidden size %d differs from the target's %d", dr->d.hidden, tg->d.hidden);
    if (block != 0 && (block < 2 || block > kMaxRows)) return fail(BVF_E_INVALID, "block %d not 0 or in [2, %d]", block, kMaxRows);
    if (n_new < 0 || n_new + block > kMaxRows) return fail(BVF_E_INVALID, "n_new %d + block %d > %d", n_new, block, kMaxRows);
    if (block == 0 && n_new == 0) return ok();
    if (n_new > 0 && !d_new_taps) return fail(BVF_E_INVALID, "d_new_taps is NULL");
    const int V = tg->d.vocab;
    if (block && (mask_token < 0 || mask_token >= V)) return fail(BVF_E_INVALID, "mask token %d outside the vocabulary", mask_token);
    if (block && !d_logits && dr->d.vocab != V) return fail(BVF_E_INVALID, "no logits buffer and the draft's scratch is sized for vocab %d", dr->d.vocab);
    const int64_t s = dr->held + n_new;
    if (s + block > dr->d.max_ctx) return fail(BVF_E_CAPACITY, "%lld context + %d block rows > max_ctx %d", (long long)s, block, dr->d.max_ctx);
    bvf_status stt = check_loaded(dr);
    if (stt) return stt;
    if (!(tg->loaded & (1u << BVF_EMBED))) return fail(BVF_E_STATE, "the target's embedding table is not loaded");
    const int H = dr->d.hidden, B = block;
    const int s_old = (int)dr->held;
    hipStream_t st = dr->st;
    if (B == 0) {
        // append only: the context rows' K/V in every draft layer, no block
        HIP_TRY(enqueue_draft_fc(dr, d_new_taps, n_new, B, st));
        uint16_t* ctx_rows = dr->act + (size_t)B * H;
        for (int l = 0; l < dr->d.n_layers; ++l) {
            Layer& L = dr->L[l];
            GemmLaunch g = gemm_for(dr, L.qkv, EPI_STORE);
            g.A = ctx_rows; g.lda = H; g.M = n_new; g.y = dr->qkv; g.ldy = L.qkv.n_out;
            HIP_TRY(launch_gemm(g, st));
            RopeAppend ra;
            ra.qkv = dr->qkv; ra.ldq = L.qkv.n_out; ra.rows_q = 0; ra.rows = n_new; ra.split_row = 0;
            ra.pos0 = s_old; ra.pos1 = s_old;
            ra.Hq = dr->d.n_q_heads; ra.nkv = L.d.n_kv_heads; ra.hd = L.d.head_dim; ra.own = 1;
            ra.qk_norm = dr->d.qk_norm; ra.q_norm = L.q_norm; ra.k_norm = L.k_norm; ra.eps = dr->d.rms_eps;
            ra.rope = L.rope; ra.plane = L.plane; ra.kv_bf16 = dr->d.kv_bf16; ra.w = L.w; ra.q_out = dr->qbuf;
            HIP_TRY(launch_rope_append(ra, st));
        }
        dr->held = s;
        return ok();
    }
    if (!dr->use_graph) {
        HIP_TRY(enqueue_draft(dr, tg, d_new_taps, n_new, d_last_token, B, embedding_scale, mask_token, d_proposals, d_logits,
                              st, nullptr));
    } else {
        // the layers' attention plans at these positions (a replay runs the plan it was captured with)
        int64_t plan = 0;
        for (int l = 0; l < dr->d.n_layers; ++l) plan = plan * 1000003 + attn_plan_key(draft_attn(dr, l, n_new, B, nullptr));
        const void* ptr[5] = {d_new_taps, d_last_token, d_proposals, d_logits, tg};
        bvf_model::DraftGraph& G = dr->dg[n_new];
        bool same = G.exec && G.plan == plan && G.block == B && G.mask == mask_token && G.scale == embedding_scale;
        for (int i = 0; i < 5 && same; ++i) same = G.ptr[i] == ptr[i];
        if (!same) {
            if (G.exec) {
                HIP_TRY(hipGraphExecDestroy(G.exec));
                G.exec = nullptr;
            }
            if (!dr->cap_st) HIP_TRY(hipStreamCreateWithFlags(&dr->cap_st, hipStreamNonBlocking));
            hipGraph_t graph = nullptr;
            HIP_TRY(hipStreamBeginCapture(dr->cap_st, hipStreamCaptureModeThreadLocal));
            hipError_t e = enqueue_draft(dr, tg, d_new_taps, n_new, d_last_token, B, embedding_scale, mask_token, d_proposals,
                                         d_logits, dr->cap_st, dr->dpos);
            hipError_t e2 = hipStreamEndCapture(dr->cap_st, &graph);
            if (e != hipSuccess || e2 != hipSuccess) {
                if (graph) (void)hipGraphDestroy(graph);
                return fail(BVF_E_DEVICE, "graph capture: %s", hipGetErrorString(e != hipSuccess ? e : e2));
            }
            e = hipGraphInstantiate(&G.exec, graph, nullptr, nullptr, 0);
            (void)hipGraphDestroy(graph);
            if (e != hipSuccess) {
                G.exec = nullptr;
                return fail(BVF_E_DEVICE, "graph instantiate: %s", hipGetErrorString(e));
            }
            G.plan = plan; G.block = B; G.mask = mask_token; G.scale = embedding_scale;
            for (int i = 0; i < 5; ++i) G.ptr[i] = ptr[i];
            ++dr->n_captures;
        }
        HIP_TRY(launch_set_i64(dr->dpos, dr->held, st));
        HIP_TRY(hipGraphLaunch(G.exec, st));
    }
    dr->held = s;
    return ok();
}

bvf_status bvf_q4_1_dequant(const bvf_model* m, int32_t layer, int32_t matrix, float* d_w) {
    if (!m || !d_w) return fail(BVF_E_INVALID, "NULL argument");
    Run r;
    bvf_status s = matrix_run(m, layer, matrix, r);
    if (s) return s;
    if (!(m->L[layer].loaded & (1u << matrix))) return fail(BVF_E_STATE, "matrix not loaded");
    HIP_TRY(launch_dequant_q4_1(r.mat->w, r.tile0, r.gu_mode, r.n_out, d_w, m->st));
    return ok();
}

bvf_status bvf_q4_1_gemm(const bvf_model* m, int32_t layer, int32_t matrix, const uint16_t* d_x, int32_t rows, float* d_y) {
    if (!m || !d_x || !d_y) return fail(BVF_E_INVALID, "NULL argument");
    if (rows < 1 || rows > m->row_cap) return fail(BVF_E_INVALID, "rows %d outside [1, %d]", rows, m->row_cap);
    Run r;
    bvf_status s = matrix_run(m, layer, matrix, r);
    if (s) return s;
    if (!(m->L[layer].loaded & (1u << matrix))) return fail(BVF_E_STATE, "matrix not loaded");
    GemmLaunch g = gemm_for(m, *r.mat, EPI_STORE);
    g.tile0 = r.tile0;
    g.tile_stride = 1;
    g.n_run_tiles = r.gu_mode ? r.mat->w.n_tiles : r.n_out / kTile;
    g.half = r.gu_mode - 1;
    g.A = d_x; g.lda = r.mat->w.K; g.M = rows; g.y = d_y; g.ldy = r.n_out;
    HIP_TRY(launch_gemm(g, m->st));
    return ok();
}

bvf_status bvf_layer_forward(bvf_model* m, int32_t layer, float* d_x, int32_t rows) {
    if (!m || !d_x) return fail(BVF_E_INVALID, "NULL argument");
    if (is_draft(m->d)) return fail(BVF_E_INVALID, "layer_forward runs verify layers");
    if (layer < 0 || layer >= m->d.n_layers) return fail(BVF_E_INVALID, "layer %d out of range", layer);
    if (rows < 1 || rows > m->row_cap) return fail(BVF_E_INVALID, "rows %d outside [1, %d]", rows, m->row_cap);
    if (m->d.ple_dim > 0)
        return fail(BVF_E_INVALID, "injected rows on a model with per-layer embeddings: its per-layer inputs need token ids");
    if (m->held + rows > m->d.max_ctx) return fail(BVF_E_CAPACITY, "positions would exceed max_ctx");
    bvf_status s = check_loaded(m);
    if (s) return s;
    HIP_TRY(launch_sumsq(d_x, m->d.hidden, rows, m->d.hidden, m->ss_x, m->st));
    HIP_TRY(run_layer(m, layer, d_x, rows, (int)m->held, nullptr, 0, nullptr));
    return ok();
}

bvf_status bvf_time_gemms(bvf_model* m, int32_t rows, int32_t iters, float* h_ms, int64_t* h_bytes) {
    if (!m || !h_ms || !h_bytes) return fail(BVF_E_INVALID, "NULL argument");
    if (is_draft(m->d)) return fail(BVF_E_INVALID, "timing runs the verify model's GEMMs");
    if (rows < 1 || rows > m->row_cap || iters < 1) return fail(BVF_E_INVALID, "rows in [1, %d], iters >= 1", m->row_cap);
    bvf_status s = check_loaded(m);
    if (s) return s;
    const int H = m->d.hidden;
    hipEvent_t e0, e1;
    HIP_TRY(hipEventCreate(&e0));
    HIP_TRY(hipEventCreate(&e1));
    for (int cls = 0; cls < 5; ++cls) {
        int64_t bytes = 0;
        int launches = 0;
        if (cls == 4 && rows > kMaxRows) {   // the bf16 head runs at most 16 rows: reported as 0
            h_ms[cls] = 0.f;
            h_bytes[cls] = 0;
            continue;
        }
        HIP_TRY(hipEventRecord(e0, m->st));
        for (int it = 0; it < iters; ++it) {
            if (cls == 4) {   // the bf16 head
                HIP_TRY(launch_head(m, nullptr, rows, m->logits_tmp, m->st, m, m->x, m->final_norm));
                bytes += (int64_t)m->d.vocab * H * 2;
                ++launches;
                continue;
            }
            for (int l = 0; l < m->d.n_layers; ++l) {
                Layer& L = m->L[l];
                GemmLaunch g;
                if (cls == 0 || cls == 2) {
                    g = gemm_for(m, cls == 0 ? L.qkv : L.gu, cls == 0 ? EPI_STORE : EPI_SWIGLU);
                    if (rows > kMaxRows) {   // wide chunks stage the bf16 rows of the separate norm
                        g.A = m->act; g.lda = H;
                    } else {
                        g.xsrc = m->x; g.ldx = H; g.ss_in = m->ss_x; g.n_ss = H / kTile;
                        g.gain = cls == 0 ? L.attn_norm : L.mlp_norm; g.eps = m->d.rms_eps;
                    }
                    if (cls == 0) { g.y = m->qkv; g.ldy = L.qkv.n_out; g.ss_out = m->ss_qkv; }
                    else { g.out = m->mbuf; g.ldo = L.d.ffn; }
                } else if (cls == 1) {
                    g = gemm_for(m, L.o, EPI_RESID); g.A = m->obuf; g.lda = L.qd; g.y = m->x; g.ldy = H; g.ss_out = m->ss_x;
                } else {
                    g = gemm_for(m, L.down, EPI_RESID); g.A = m->mbuf; g.lda = L.d.ffn; g.y = m->x; g.ldy = H; g.ss_out = m->ss_x;
                }
                g.M = rows;
                HIP_TRY(launch_gemm(g, m->st));
                bytes += (int64_t)g.w.n_tiles * g.w.G * (1024 + 256);
                ++launches;
            }
        }
        HIP_TRY(hipEventRecord(e1, m->st));
        HIP_TRY(hipEventSynchronize(e1));
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, e0, e1));
        h_ms[cls] = ms / launches;
        h_bytes[cls] = bytes / launches;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return ok();
}

bvf_status bvf_pass_bytes(const bvf_model* m, int64_t* q4, int64_t* head) {
    if (!m || !q4 || !head) return fail(BVF_E_INVALID, "NULL argument");
    int64_t b = 0;
    for (const Layer& L : m->L)
        for (const Mat* M : {&L.qkv, &L.o, &L.gu, &L.down, &L.ple_gate, &L.ple_proj})
            b += (int64_t)M->w.n_tiles * M->w.G * (1024 + 256);
    *q4 = b;
    *head = is_draft(m->d) ? 0 : (int64_t)m->d.vocab * m->d.hidden * 2;
    return ok();
}

}  // extern "C"
