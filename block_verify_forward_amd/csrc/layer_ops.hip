// gfx950 kernels of the verify pass other than the weight-streaming GEMM: Q4_1 repack and debug
// dequant, RoPE table, embedding gather, RMSNorm, QK-norm + RoPE + KV append, GQA block attention
// over the per-layer KV planes, argmax + greedy accept.
#include "bvf_impl.hpp"

#include <algorithm>
#include <cmath>
#include <mutex>

namespace bvf {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32; NaN stays a NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// Orders this wave's LDS writes before its later LDS reads by other lanes (each wave owns its own
// LDS slice, so no workgroup barrier is needed; waves of a workgroup run different key ranges).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier over LDS traffic only: this wave's LDS reads and writes are complete, then
// s_barrier. (__syncthreads also waits for every outstanding global load, which would wait for the
// next sub-chunk's K/V copies.)
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt for at most N vector memory operations of this wave in flight (LDS and scalar counts
// untouched)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}


// Reductions over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15) without LDS traffic: quad
// swaps, then the half-row and row mirrors; every lane ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));    // lane ^ 1
    v = fmaxf(v, dpp<0x4E>(v));    // lane ^ 2
    v = fmaxf(v, dpp<0x141>(v));   // row_half_mirror
    v = fmaxf(v, dpp<0x140>(v));   // row_mirror
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    return v;
}

// Reductions over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48) with the
// row swaps of gfx950: v_permlane16_swap exchanges the odd rows of its first register with the even
// rows of its second, v_permlane32_swap the upper half of the first with the lower half of the
// second. Given two copies of a value, each lane then holds its own value and its partner's, in
// the same order on both partners, so both compute the same bits. The swaps are written as inline
// asm with both registers as outputs: this compiler's builtins return the first register for both
// results. The s_nop pairs cover the VALU hazards around the swap.
__device__ __forceinline__ void swap_rows16(float& x, float& y) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void swap_rows32(float& x, float& y) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ float swap_rows16_max(float v) { float x = v, y = v; swap_rows16(x, y); return fmaxf(x, y); }
__device__ __forceinline__ float swap_rows32_max(float v) { float x = v, y = v; swap_rows32(x, y); return fmaxf(x, y); }
__device__ __forceinline__ float swap_rows16_sum(float v) { float x = v, y = v; swap_rows16(x, y); return x + y; }
__device__ __forceinline__ float swap_rows32_sum(float v) { float x = v, y = v; swap_rows32(x, y); return x + y; }
__device__ __forceinline__ float rows4_max(float v) { return swap_rows32_max(swap_rows16_max(v)); }
__device__ __forceinline__ float rows4_sum(float v) { return swap_rows32_sum(swap_rows16_sum(v)); }
// all 64 lanes: the 16 lanes of each row, then the four rows
__device__ __forceinline__ float wave64_max(float v) { return rows4_max(row16_max(v)); }
__device__ __forceinline__ float wave64_sum(float v) { return rows4_sum(row16_sum(v)); }

// N consecutive floats (N a multiple of 4, or 2) through 16- or 8-byte accesses; the addresses are
// aligned to the access size.
template <int N>
__device__ __forceinline__ void load_vec(float* v, const float* p) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 t = *(const float4*)(p + i);
            v[i] = t.x; v[i + 1] = t.y; v[i + 2] = t.z; v[i + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 2) {
            const float2 t = *(const float2*)(p + i);
            v[i] = t.x; v[i + 1] = t.y;
        }
    }
}
template <int N>
__device__ __forceinline__ void store_vec(float* p, const float* v) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) *(float4*)(p + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 2) *(float2*)(p + i) = make_float2(v[i], v[i + 1]);
    }
}
// N consecutive bf16 (N a multiple of 2) as floats
template <int N>
__device__ __forceinline__ void load_bf16_vec(float* v, const uint16_t* p) {
    if constexpr (N % 8 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 8) {
            const uint4 t = *(const uint4*)(p + i);
            const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[i + 2 * q] = __builtin_bit_cast(float, w[q] << 16);
                v[i + 2 * q + 1] = __builtin_bit_cast(float, w[q] & 0xffff0000u);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 2) {
            const uint32_t w = *(const uint32_t*)(p + i);
            v[i] = __builtin_bit_cast(float, w << 16);
            v[i + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
        }
    }
}

// N consecutive bf16 (N even; the address aligned to the access) as raw 32-bit pairs, and their widening: a load whose
// conversion is placed later does not make the wave wait for it at the load site
template <int N>
__device__ __forceinline__ void load_bf16_raw(uint32_t* w, const uint16_t* p) {
    if constexpr (N % 8 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 8) {
            const uint4 t = *(const uint4*)(p + i);
            w[i / 2] = t.x; w[i / 2 + 1] = t.y; w[i / 2 + 2] = t.z; w[i / 2 + 3] = t.w;
        }
    } else if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const uint2 t = *(const uint2*)(p + i);
            w[i / 2] = t.x; w[i / 2 + 1] = t.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 2) w[i / 2] = *(const uint32_t*)(p + i);
    }
}
template <int N>
__device__ __forceinline__ void widen_bf16(float* v, const uint32_t* w) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ---------------------------------------------------------------------------------------------
// Q4_1 repack: canonical host blocks -> the column-tiled image the GEMM streams (one thread per
// 32-weight block). Canonical block ([CARD], "Weights" row; byte order fixed by the header):
// fp16 scale, fp16 min, 16 code bytes, code j < 16 in the low nibble of byte j, j + 16 in the high.
// gu_mode: 0 plain (column col0 + n), 1 gate (tile n / 8, column n % 8), 2 up (column 8 + n % 8).
// ---------------------------------------------------------------------------------------------
__global__ void k_repack(const uint8_t* __restrict__ canon, int n_out, int nb, uint8_t* __restrict__ codes,
                         uint8_t* __restrict__ sm, int G, int col0, int gu_mode) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)n_out * nb) return;
    const int n = (int)(idx / nb), b = (int)(idx % nb);
    const uint32_t* blk = (const uint32_t*)(canon + idx * 20);   // 20-byte blocks are 4-byte aligned
    uint32_t w[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) w[i] = blk[i];
    int T, c;
    if (gu_mode == 0) {
        T = (col0 + n) >> 4;
        c = (col0 + n) & 15;
    } else {
        T = n >> 3;
        c = (n & 7) + (gu_mode == 2 ? 8 : 0);
    }
    const int g = b >> 2, j = b & 3;
    const uint8_t* q8 = (const uint8_t*)&w[1];
    for (int sub = 0; sub < 4; ++sub) {
        uint32_t d = 0;
        for (int e = 0; e < 8; ++e) {
            const int kb = 8 * sub + e;
            const uint32_t q = kb < 16 ? (q8[kb] & 15u) : (q8[kb - 16] >> 4);
            d |= q << (4 * ((e >> 1) + 4 * (e & 1)));
        }
        ((uint32_t*)codes)[(((size_t)T * G + g) * 64 + sub * 16 + c) * 4 + j] = d;
    }
    ((uint32_t*)sm)[(((size_t)T * G + g) * 16 + c) * 4 + j] = w[0];   // scale | min << 16
}

// fp32 weights of one matrix from the packed image: weight = fma(scale, code, min), one rounding
// of the exact value scale * code + min.
__global__ void k_dequant(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ sm, int G, int tile0,
                          int gu, int n_out, int n_in, float* __restrict__ out) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)n_out * n_in) return;
    const int n = (int)(idx / n_in), k = (int)(idx % n_in);
    const int T = gu ? (n >> 3) : tile0 + (n >> 4);
    const int c = gu ? (n & 7) + (gu == 2 ? 8 : 0) : (n & 15);
    const int g = k >> 7, j = (k >> 5) & 3, kb = k & 31, sub = kb >> 3, e = kb & 7;
    const uint32_t d = ((const uint32_t*)codes)[(((size_t)T * G + g) * 64 + sub * 16 + c) * 4 + j];
    const uint32_t q = (d >> (4 * ((e >> 1) + 4 * (e & 1)))) & 15u;
    const uint32_t s = ((const uint32_t*)sm)[(((size_t)T * G + g) * 16 + c) * 4 + j];
    const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(s & 0xffffu));
    const float mn = (float)__builtin_bit_cast(_Float16, (uint16_t)(s >> 16));
    out[idx] = fmaf(sc, (float)q, mn);
}

// RoPE table [max_ctx][hd / 2] of (cos, sin) of p * base^(-2i / hd), evaluated in double.
__global__ void k_rope_table(float2* table, int max_ctx, int hd, double base) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int h = hd / 2;
    if (idx >= (size_t)max_ctx * h) return;
    const int p = (int)(idx / h), i = (int)(idx % h);
    const double th = (double)p * pow(base, -2.0 * i / hd);
    table[idx] = make_float2((float)cos(th), (float)sin(th));
}

// x[r][:] = E[token_r] * scale (fp32). fill_token >= 0: row 0 takes tokens[0], the other rows
// fill_token (the draft block). Token ids outside [0, V) are clamped. ss (optional): per row and
// 16-column tile, the sum of squares of x (what the next GEMM's folded RMSNorm reads).
__global__ void k_embed(const int32_t* __restrict__ tokens, int fill_token, const uint16_t* __restrict__ E, int V,
                        int H, float scale, float* __restrict__ x, float* __restrict__ ss) {
    const int r = blockIdx.y;
    int t = (fill_token >= 0 && r > 0) ? fill_token : tokens[fill_token >= 0 ? 0 : r];
    t = t < 0 ? 0 : (t >= V ? V - 1 : t);
    const int i = blockIdx.x * blockDim.x + threadIdx.x;   // grid covers H exactly (H % 256 == 0 ... or masked)
    const float v = i < H ? bf16_to_f32(E[(size_t)t * H + i]) * scale : 0.f;
    if (i < H) x[(size_t)r * H + i] = v;
    if (ss) {
        float q = v * v;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) q += __shfl_xor(q, o);
        if ((i & 15) == 0 && i < H) ss[(size_t)r * (H / 16) + i / 16] = q;
    }
}

// ss[r][j] = sum of x[r][16 j .. 16 j + 15]^2
__global__ void k_sumsq(const float* __restrict__ x, int ldx, int H, float* __restrict__ ss) {
    const int r = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const float v = i < H ? x[(size_t)r * ldx + i] : 0.f;
    float q = v * v;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) q += __shfl_xor(q, o);
    if ((i & 15) == 0 && i < H) ss[(size_t)r * (H / 16) + i / 16] = q;
}

// out[r][i] = bf16(x[r][i] / sqrt(mean_i x[r][i]^2 + eps) * g[i]); one workgroup per row.
// One 256-thread block per row: every float4 of the row and its four gains are loaded before the
// sum of squares (rows of up to 8192 values stay in registers, so the output needs no second read;
// longer rows continue in a loop), then bf16(x * inv * gain) is written four values at a time.
constexpr int kNormPieces = 8;   // float4 pieces per thread held in registers
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ x, int ldx, int H,
                                                 const uint16_t* __restrict__ g, float eps, uint16_t* __restrict__ out,
                                                 int ldo) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    const float* xr = x + (size_t)r * ldx;
    uint16_t* orow = out + (size_t)r * ldo;
    float4 v[kNormPieces];
    uint2 gv[kNormPieces];   // the gains of the same pieces, loaded in the same round
#pragma unroll
    for (int j = 0; j < kNormPieces; ++j) {
        const int i = 4 * threadIdx.x + 1024 * j;
        v[j] = i < H ? *(const float4*)(xr + i) : make_float4(0.f, 0.f, 0.f, 0.f);
        gv[j] = i < H ? *(const uint2*)(g + i) : make_uint2(0u, 0u);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kNormPieces; ++j) ss += (v[j].x * v[j].x + v[j].y * v[j].y) + (v[j].z * v[j].z + v[j].w * v[j].w);
    for (int i = 4 * threadIdx.x + 1024 * kNormPieces; i < H; i += 1024) {
        const float4 t = *(const float4*)(xr + i);
        ss += (t.x * t.x + t.y * t.y) + (t.z * t.z + t.w * t.w);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = red[0] + red[1] + red[2] + red[3];
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
    auto put = [&](int i, const float4& t, const uint2& gw) {
        const float g0 = __builtin_bit_cast(float, gw.x << 16), g1 = __builtin_bit_cast(float, gw.x & 0xffff0000u);
        const float g2 = __builtin_bit_cast(float, gw.y << 16), g3 = __builtin_bit_cast(float, gw.y & 0xffff0000u);
        *(uint2*)(orow + i) = make_uint2(pack_bf16x2(t.x * inv * g0, t.y * inv * g1), pack_bf16x2(t.z * inv * g2, t.w * inv * g3));
    };
#pragma unroll
    for (int j = 0; j < kNormPieces; ++j) {
        const int i = 4 * threadIdx.x + 1024 * j;
        if (i < H) put(i, v[j], gv[j]);
    }
    for (int i = 4 * threadIdx.x + 1024 * kNormPieces; i < H; i += 1024) put(i, *(const float4*)(xr + i), *(const uint2*)(g + i));
}

// One wave per (row, head): per-head RMSNorm (optional), rotate-half RoPE at the row's position;
// q heads go to q_out, k/v heads of an own layer are written into the plane at the position.
__global__ __launch_bounds__(64) void k_rope_append(RopeAppend a) {
    const int row = blockIdx.x, head = blockIdx.y, lane = threadIdx.x;
    const int hd = a.hd, h2 = hd / 2;
    const int p = row < a.split_row ? a.pos0 + row : a.pos1 + (row - a.split_row);
    const float* src;
    float* dst = nullptr;        // q heads, or a K row of an fp32 plane
    uint16_t* dst16 = nullptr;   // a K row of a bf16 plane
    const uint16_t* gain;
    const int qd = a.Hq * hd, kvd = a.nkv * hd;
    if (head < a.Hq) {
        if (row >= a.rows_q) return;
        src = a.qkv + (size_t)row * a.ldq + head * hd;
        dst = a.q_out + ((size_t)row * a.Hq + head) * hd;
        gain = a.q_norm;
    } else {
        if (!a.own || row >= a.rows) return;
        const int gh = head - a.Hq;
        src = a.qkv + (size_t)row * a.ldq + qd + gh * hd;
        gain = a.k_norm;
        const float* vs = a.qkv + (size_t)row * a.ldq + qd + kvd + gh * hd;
        const size_t off = (size_t)p * 2 * a.w;
        if (a.kv_bf16) {
            uint16_t* prow = (uint16_t*)a.plane + off;
            dst16 = prow + gh * hd;
            for (int i = lane; i < hd; i += 64) prow[a.w + gh * hd + i] = f32_to_bf16(vs[i]);
        } else {
            float* prow = (float*)a.plane + off;
            dst = prow + gh * hd;
            for (int i = lane; i < hd; i += 64) prow[a.w + gh * hd + i] = vs[i];
        }
    }
    float lo[4], hi[4];
    float ss = 0.f;
    const int per = (h2 + 63) / 64;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int i = lane + 64 * t;
        lo[t] = (t < per && i < h2) ? src[i] : 0.f;
        hi[t] = (t < per && i < h2) ? src[i + h2] : 0.f;
        ss = fmaf(lo[t], lo[t], fmaf(hi[t], hi[t], ss));
    }
    float inv = 1.f;
    if (a.qk_norm) inv = 1.0f / sqrtf(wave_sum(ss) / (float)hd + a.eps);
    const float2* rt = a.rope + (size_t)p * h2;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int i = lane + 64 * t;
        if (t >= per || i >= h2) continue;
        float x0 = lo[t] * inv, x1 = hi[t] * inv;
        if (a.qk_norm) {
            x0 *= bf16_to_f32(gain[i]);
            x1 *= bf16_to_f32(gain[i + h2]);
        }
        const float2 cs = rt[i];
        const float y0 = x0 * cs.x - x1 * cs.y, y1 = x0 * cs.y + x1 * cs.x;
        if (dst16) {
            dst16[i] = f32_to_bf16(y0);
            dst16[i + h2] = f32_to_bf16(y1);
        } else {
            dst[i] = y0;
            dst[i + h2] = y1;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// GQA block attention, one kernel per layer ([PR2303] "What changes": a KV-shared layer reads its
// owner's cache and appends nothing). A workgroup owns 16 query vectors (qv = m * Hg + head in the
// group) of one KV head g and one chunk of keys:
//   1. the 16 queries: per-head RMSNorm (sums of squares from the q|k|v GEMM's epilogue) and
//      rotate-half RoPE at the row's position, into LDS;
//   2. on an own layer, the chunk's new rows (the rows of this pass): K normalised and rotated, V
//      copied, appended to the plane at their positions;
//   3. each of the 4 waves runs 16 keys per step with fp32 MFMA (v_mfma_f32_16x16x4_f32):
//      S = Q K^T, online softmax, O += P V (P through LDS to the A layout, V rows staged in LDS);
//   4. the waves merge (max, sum, O) in LDS and the workgroup stores its chunk's partial;
//      k_attn_combine then merges the chunks in chunk order and writes bf16 O.
// Row m (position pos(m)) sees keys [max(0, pos - window + 1), pos] (causal; window 0 = all) or,
// in a draft block, [ctx_lo, ctx_hi].
// ---------------------------------------------------------------------------------------------
constexpr int kKeysPerStep = 16;

struct AttnK {
    const float* qkv;        // [rows][ldq] raw q | k | v (GEMM output)
    const float* ss;         // [rows][ldq / 16] per-tile sums of squares of qkv
    int ldq;
    const uint16_t* q_norm;
    const uint16_t* k_norm;
    int qk_norm;
    float eps;
    const float2* rope;      // [max_ctx][hd / 2]
    void* plane;             // own or owner's plane [max_ctx][2][w], fp32 or (kv_bf16) bf16 values
    int kv_bf16;
    int ring_cap;            // > 0: ring plane of ring_cap slots (position p in slot p mod ring_cap)
    int w, own;
    int M, Hq, nkv, Hg, NQ, n_qt;
    int causal, pos0, window, ctx_lo, ctx_hi;
    int np0, np1, sp, r_lo, r_hi;   // new rows: positions [np0, np1); row of p: p < sp ? r_lo + p - np0 : r_hi + p - sp
    int key_lo, n_keys, spw, n_chunks;   // keys [key_lo, key_lo + n_keys); spw sub-chunks per workgroup
    const int64_t* dpos;     // graph replays: positions held read here (see bind_positions)
    int n_ctx;               // draft block replays: context rows appended before the block rows
    float* part;             // [n_qt][nkv][n_chunks][16][attn_part_ld(hd)] partials: O, then max and sum
    int* counters;           // [n_qt * nkv]
    uint16_t* out;           // [M][Hq * hd] bf16
};

// A pass captured in a graph reads the positions held P from device memory.
// Causal: its rows sit at P .. P + M - 1, an own layer appends them, and row m sees
// [max(0, P + m - window + 1), P + m].
// Draft block: the n_ctx context rows go to P .. s - 1 (s = P + n_ctx) and the M block rows to
// s .. s + M - 1; every block row sees [max(0, s - window), s + M - 1] (window: the draft's context
// window, 0 = all), and the key range also covers the appended context rows.
__device__ __forceinline__ void bind_positions(AttnK& a) {
    const int P = (int)*a.dpos;
    if (a.causal) {
        a.pos0 = P;
        a.np0 = P;
        a.np1 = P + a.M;
        a.sp = P;
        const int lo = (a.window > 0 && P - a.window + 1 > 0) ? P - a.window + 1 : 0;
        a.key_lo = lo;
        a.n_keys = P + a.M - lo;
        return;
    }
    const int s = P + a.n_ctx;
    a.pos0 = s;
    a.ctx_lo = (a.window > 0 && s - a.window > 0) ? s - a.window : 0;
    a.ctx_hi = s + a.M - 1;
    a.np0 = P;
    a.np1 = s + a.M;
    a.sp = s;
    const int lo = a.own && a.ctx_lo > P ? P : a.ctx_lo;
    a.key_lo = lo;
    a.n_keys = s + a.M - lo;
}

__global__ void k_set_i64(int64_t* dst, int64_t v) { *dst = v; }

// Plane slot of position p: p itself, or p mod the ring's capacity on a ring plane.
__device__ __forceinline__ int kv_slot(const AttnK& a, int p) { return a.ring_cap > 0 ? p % a.ring_cap : p; }

__device__ __forceinline__ void row_range(const AttnK& a, int m, int& lo, int& hi) {
    if (a.causal) {
        hi = a.pos0 + m;
        lo = (a.window > 0 && hi - a.window + 1 > 0) ? hi - a.window + 1 : 0;
    } else {
        lo = a.ctx_lo;
        hi = a.ctx_hi;
    }
}

// sum of squares of a head (hd columns from column c0 of row r) from the per-tile partials
__device__ __forceinline__ float head_ss(const AttnK& a, int r, int c0, int hd) {
    float q = 0.f;
    const float* p = a.ss + (size_t)r * (a.ldq / 16) + c0 / 16;
    for (int i = 0; i < hd / 16; ++i) q += p[i];
    return q;
}

// Keys per sub-chunk: the K and V tiles of a sub-chunk take 16 KB each in LDS with fp32 planes (16
// keys at hd 256: small chunks spread the K/V reads over many compute units), at least one 16-key
// MFMA block.
__host__ __device__ constexpr int attn_ck(int hd) { return 4096 / hd > 16 ? 4096 / hd : 16; }

// LDS of k_attention<hd, kvb, multi>: the K and V tiles (padded rows), the query rows (with multi:
// the larger of them and a second K/V stage) and the partial scores (the arrays declared in the
// kernel).
constexpr size_t attn_lds_bytes(int hd, bool kvb, bool multi) {
    const size_t ck = attn_ck(hd), eb = kvb ? 2 : 4;
    const size_t kv = ck * (hd + 16 / eb) * eb + ck * (hd + 16) * eb, q = (size_t)16 * (hd + 4) * 4;
    return kv + (multi && kv > q ? kv : q) + (size_t)4 * 16 * (ck + 4) * 4;
}

// Tile element of the K/V planes: fp32, or (KVB) bf16 values widened exactly where they are read.
template <bool KVB> struct KVElem { using T = float; };
template <> struct KVElem<true> { using T = uint16_t; };

template <int N>
__device__ __forceinline__ void store_bf16_vec(uint16_t* p, const float* v) {
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    if constexpr (N % 8 == 0) {
#pragma unroll
        for (int i = 0; i < N / 2; i += 4) *(uint4*)(p + 2 * i) = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
    } else if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 2; i += 2) *(uint2*)(p + 2 * i) = make_uint2(w[i], w[i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) *(uint32_t*)(p + 2 * i) = w[i];
    }
}

// One workgroup per (key chunk, KV head, tile of 16 query vectors). The chunk's keys go through LDS
// in sub-chunks of CK keys.
// MULTI (long key ranges): several sub-chunks per workgroup through two LDS stages, the copies of
// the next sub-chunk in flight while the current one is computed. The query values are read into
// registers once, and the space of the query rows then holds the second stage, so a workgroup takes
// ~73 KB of LDS at head dim 256 with fp32 planes and two workgroups share a compute unit.
// Without MULTI: one sub-chunk, no loop; its K/V copies are issued before any other load.
// KVB: the planes hold bf16 values; the tiles keep them as bf16 and the reads widen them (exact),
// and new rows are written rounded to the plane and the tile, so every K/V value the scores and
// PV see is the stored one.
template <int HD, bool KVB, bool MULTI>
__global__ __launch_bounds__(256) void k_attention(AttnK a) {
    using TT = typename KVElem<KVB>::T;
    constexpr int CK = attn_ck(HD);      // keys per sub-chunk
    constexpr int KB = CK / 16;          // 16-key blocks per sub-chunk
    constexpr int DW = HD / 4;           // dims owned by each wave (scores over them, then O for them)
    constexpr int H2 = HD / 2;
    constexpr int PPT = H2 / 16;         // rotate-half pairs per thread (16 threads per vector)
    static_assert(HD <= 256, "a head's tile sums of squares: at most one per thread of a vector");
    constexpr int EPU = 16 / (int)sizeof(TT);   // values per 16-byte copy unit
    constexpr int UPR = HD / EPU;               // copy units per K or V row
    // padded rows: K rows shift by 16 bytes (the 16 rows of a score read hit distinct banks), V rows
    // by 64 bytes (fp32) or 32 bytes (bf16) (the 4 rows x 16 dims of a PV read hit distinct banks)
    constexpr int LDK = HD + 16 / (int)sizeof(TT);
    constexpr int LDV = HD + (KVB ? 16 : 16);
    constexpr int LD = HD + 4;           // query rows
    constexpr size_t KT_BYTES = (size_t)CK * LDK * sizeof(TT), VT_BYTES = (size_t)CK * LDV * sizeof(TT);
    constexpr size_t Q_BYTES = (size_t)16 * LD * 4;
    constexpr size_t ST1 = MULTI && KT_BYTES + VT_BYTES > Q_BYTES ? KT_BYTES + VT_BYTES : Q_BYTES;
    static_assert(KT_BYTES % 16 == 0, "the second stage's V rows start 16-byte aligned");
    __shared__ __attribute__((aligned(16))) TT K0[CK][LDK];
    __shared__ __attribute__((aligned(16))) TT V0[CK][LDV];
    // the query rows; with MULTI, after they are read into registers, the second K/V stage
    __shared__ __attribute__((aligned(16))) uint8_t st1[ST1];
    __shared__ __attribute__((aligned(16))) float Sp[4][16][CK + 4];   // per-wave partial scores (over the wave's dims)
    float (*Qs)[LD] = reinterpret_cast<float (*)[LD]>(st1);
    TT (*K1)[LDK] = reinterpret_cast<TT (*)[LDK]>(st1);
    TT (*V1)[LDV] = reinterpret_cast<TT (*)[LDV]>(st1 + KT_BYTES);
    constexpr int NPW = 2 * CK / 4;   // K/V copy instructions per wave per stage
    if (a.dpos) bind_positions(a);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    // block order: the query tiles of one (chunk, KV head) pair sit 8 blocks apart, so they run on
    // the same XCD at about the same time and the second tile's K/V copies find the rows in its L2;
    // the grid is padded to whole groups of 8 pairs and the padding blocks leave at once
    const int xl = blockIdx.x % 8, rest = blockIdx.x / 8;
    const int qt = rest % a.n_qt, pidx = (rest / a.n_qt) * 8 + xl;
    if (pidx >= a.n_chunks * a.nkv) return;   // uniform in the workgroup
    const int chunk = pidx % a.n_chunks;
    const int g = pidx / a.n_chunks;
    const int col = lane & 15, grp = lane >> 4;
    const int qd = a.Hq * HD;
    const size_t prow = (size_t)2 * a.w;
    const int wk0 = a.key_lo + chunk * a.spw * CK;                   // this workgroup's keys [wk0, wk1)
    const int wk1 = min(a.key_lo + a.n_keys, wk0 + a.spw * CK);

    // K and V rows of a sub-chunk: direct global->LDS copies, one row (UPR <= 64 16-byte units) per
    // instruction, CK / 4 rows per wave (rows wave + 4 t); rows past c1 repeat row c0 (finite;
    // masked below). A sub-chunk past the workgroup's keys (c0 >= wk1: the two-stage loop's last
    // copies, never read) copies row wk1 - 1 into every row. The ring slot of each row steps by 4
    // from the first one, so the copies form one straight run of NPW instructions with no branch
    // between them: the compiler's wait-count analysis then sees the same copies on every path and
    // needs no wait of its own before the reads of the other stage.
    static_assert(UPR <= 64, "one copy instruction per row");
    auto issue_kv = [&](TT (*Kt)[LDK], TT (*Vt)[LDV], int c0) __attribute__((always_inline)) {
        const int c1 = min(wk1, c0 + CK);
        const int cb = c0 < wk1 ? c0 : wk1 - 1;   // the row repeated past c1
        const int rc = a.ring_cap;
        const int sb = rc > 0 ? cb % rc : cb;     // its plane slot
        int sl = rc > 0 ? (cb + wave) % rc : cb + wave;   // slot of row wave (when it is a key)
        static_assert(CK % 4 == 0, "K (and V) copies split evenly over the 4 waves");
        int slots[CK / 4];
#pragma unroll
        for (int t = 0; t < CK / 4; ++t) {
            slots[t] = c0 + wave + 4 * t < c1 ? sl : sb;
            sl += 4;
            sl = rc > 0 && sl >= rc ? sl - rc : sl;   // one wrap: a ring holds at least 4 slots
        }
        const int unit = lane;
#pragma unroll
        for (int kv = 0; kv < 2; ++kv)
#pragma unroll
            for (int t = 0; t < CK / 4; ++t) {
                const int kk = wave + 4 * t;
                if (UPR == 64 || unit < UPR) {
                    const size_t e = (size_t)slots[t] * prow + (size_t)kv * a.w + g * HD + unit * EPU;
                    const void* src = (const TT*)a.plane + e;
                    void* dst = kv ? (void*)&Vt[kk][0] : (void*)&Kt[kk][0];
                    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
                }
            }
    };

    // new rows of an own layer (16 threads per row): raw K, V, RoPE row and the head's sums of
    // squares into registers; store_row normalises, rotates and writes them to LDS and the plane
    const int ri = tid >> 4, jr = tid & 15;
    float kr0[PPT], kr1[PPT], vr0[PPT], vr1[PPT], ssr = 0.f;
    float2 csr[PPT];
    uint32_t gkw0[PPT / 2], gkw1[PPT / 2];   // the K gains, raw (widened in store_row)
    // has == false: the thread has no row; it loads row 0 at position 0 (readable, unused), so the
    // loads need no branch (a load under a branch is waited for where the branches join)
    auto load_row = [&](int p, bool has = true) __attribute__((always_inline)) {
        const int r = !has ? 0 : p < a.sp ? a.r_lo + (p - a.np0) : a.r_hi + (p - a.sp);
        if (!has) p = 0;
        const float* ks = a.qkv + (size_t)r * a.ldq + qd + g * HD;
        const float* vs = a.qkv + (size_t)r * a.ldq + qd + a.nkv * HD + g * HD;
        const float2* rt = a.rope + (size_t)p * H2;
        const int d0 = jr * PPT;
        load_vec<PPT>(kr0, ks + d0);
        load_vec<PPT>(kr1, ks + d0 + H2);
        load_vec<PPT>(vr0, vs + d0);
        load_vec<PPT>(vr1, vs + d0 + H2);
        load_vec<2 * PPT>((float*)csr, (const float*)(rt + d0));
        // the head's tile sums (one per thread jr < HD / 16), loaded without a branch and selected
        // where they are used (store_row)
        ssr = *(a.qk_norm && jr < HD / 16 ? a.ss + (size_t)r * (a.ldq / 16) + (qd + g * HD) / 16 + jr
                                           : (const float*)a.rope);
        // the K gains with the row (no round trip of their own in store_row); without QK-norm they
        // read the RoPE table (unused)
        const uint16_t* gks = a.qk_norm ? a.k_norm : (const uint16_t*)a.rope;
        load_bf16_raw<PPT>(gkw0, gks + d0);
        load_bf16_raw<PPT>(gkw1, gks + d0 + H2);
    };
    auto store_row = [&](int p, int c0, TT (*Kt)[LDK], TT (*Vt)[LDV]) __attribute__((always_inline)) {
        const float ssv = a.qk_norm && jr < HD / 16 ? ssr : 0.f;
        const float inv = a.qk_norm ? 1.0f / sqrtf(row16_sum(ssv) / (float)HD + a.eps) : 1.f;
        const size_t prow_off = (size_t)kv_slot(a, p) * prow + g * HD;
        const int kk = p - c0;
        const int d0 = jr * PPT;
        float gk0[PPT], gk1[PPT], k0[PPT], k1[PPT];
        if (a.qk_norm) {
            widen_bf16<PPT>(gk0, gkw0);
            widen_bf16<PPT>(gk1, gkw1);
        } else {
#pragma unroll
            for (int i = 0; i < PPT; ++i) gk0[i] = gk1[i] = 1.f;
        }
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const float y0 = kr0[i] * inv * gk0[i], y1 = kr1[i] * inv * gk1[i];
            k0[i] = y0 * csr[i].x - y1 * csr[i].y;
            k1[i] = y0 * csr[i].y + y1 * csr[i].x;
        }
        TT* dst = (TT*)a.plane + prow_off;
        // every query tile of the chunk computes the rows for its own stage; tile 0 writes the plane
        const bool to_plane = qt == 0;
        if constexpr (KVB) {   // the plane and the tile take the same rounded values
            if (to_plane) {
                store_bf16_vec<PPT>(dst + d0, k0);
                store_bf16_vec<PPT>(dst + d0 + H2, k1);
                store_bf16_vec<PPT>(dst + a.w + d0, vr0);
                store_bf16_vec<PPT>(dst + a.w + d0 + H2, vr1);
            }
            store_bf16_vec<PPT>(&Kt[kk][d0], k0);
            store_bf16_vec<PPT>(&Kt[kk][d0 + H2], k1);
            store_bf16_vec<PPT>(&Vt[kk][d0], vr0);
            store_bf16_vec<PPT>(&Vt[kk][d0 + H2], vr1);
        } else {
            if (to_plane) {
                store_vec<PPT>(dst + d0, k0);
                store_vec<PPT>(dst + d0 + H2, k1);
                store_vec<PPT>(dst + a.w + d0, vr0);
                store_vec<PPT>(dst + a.w + d0 + H2, vr1);
            }
            store_vec<PPT>(&Kt[kk][d0], k0);
            store_vec<PPT>(&Kt[kk][d0 + H2], k1);
            store_vec<PPT>(&Vt[kk][d0], vr0);
            store_vec<PPT>(&Vt[kk][d0 + H2], vr1);
        }
    };
    auto new_rows = [&](int c0, int& p_lo, int& p_hi) {
        const int c1 = min(wk1, c0 + CK);
        p_lo = a.own ? max(c0, a.np0) : 0;
        p_hi = a.own ? min(c1, a.np1) : 0;
    };

    // 1. the 16 query vectors of the tile: per-head RMSNorm (sums of squares from the q|k|v GEMM's
    //    epilogue) and rotate-half RoPE at the row's position, into LDS; 16 threads per vector.
    //    Their loads, and (one sub-chunk) those of its new rows, go out before the K/V copies
    //    (a wave's loads return in order: the query is built while the copies are in flight), and
    //    nothing waits for a load before the copies are issued: the gains stay raw and the first
    //    sum-of-squares term is taken as is.
    {
        const int qi = tid >> 4, j = tid & 15;
        const int qv = qt * 16 + qi;
        const bool live = qv < a.NQ;
        const int m = live ? qv / a.Hg : 0, h = live ? g * a.Hg + qv % a.Hg : 0;
        const float* src = a.qkv + (size_t)m * a.ldq + h * HD;
        const float2* rt = a.rope + (size_t)(a.pos0 + m) * H2;
        float x0[PPT], x1[PPT], g0[PPT], g1[PPT];
        uint32_t gw0[PPT / 2], gw1[PPT / 2];
        float2 cs[PPT];
        const int d0 = j * PPT;   // this thread's PPT consecutive pairs (d0 + i, d0 + i + H2)
        load_vec<PPT>(x0, src + d0);
        load_vec<PPT>(x1, src + d0 + H2);
        load_vec<2 * PPT>((float*)cs, (const float*)(rt + d0));
        // without QK-norm the gain loads read the RoPE table (any HD readable halves; unused)
        const uint16_t* gsrc = a.qk_norm ? a.q_norm : (const uint16_t*)a.rope;
        load_bf16_raw<PPT>(gw0, gsrc + d0);
        load_bf16_raw<PPT>(gw1, gsrc + d0 + H2);
        // the head's HD / 16 <= 16 tile sums: one per thread j < HD / 16, loaded without a branch
        // (a load under a branch is waited for where the branches join)
        const bool has_ss = a.qk_norm && j < HD / 16;
        const float ssq_raw = *(has_ss ? a.ss + (size_t)m * (a.ldq / 16) + h * (HD / 16) + j : (const float*)a.rope);
        // the first sub-chunk's new rows (the two-stage form loads them where it stores them: only
        // the workgroup that holds the pass's positions has any). With fp32 planes only waves with
        // a new row issue the loads; with bf16 planes every thread does (rows of no one read row 0
        // at position 0), since the compiler would otherwise round the V rows to bf16 inside the
        // branch and wait for them there, before the copies. (Issuing them after the copies instead
        // made the query wait for the copies, with the same step time.)
        if constexpr (!MULTI) {
            int p_lo, p_hi;
            new_rows(wk0, p_lo, p_hi);
            if constexpr (KVB) load_row(p_lo + ri, p_lo + ri < p_hi);
            else if (p_lo + ri < p_hi) load_row(p_lo + ri);
        }
        asm volatile("" ::: "memory");   // these loads leave before the K/V copies
        __builtin_amdgcn_sched_barrier(0);
        if (wk0 < wk1) issue_kv(K0, V0, wk0);
        widen_bf16<PPT>(g0, gw0);
        widen_bf16<PPT>(g1, gw1);
        if (!a.qk_norm) {
#pragma unroll
            for (int i = 0; i < PPT; ++i) g0[i] = g1[i] = 1.f;
        }
        const float ssq = has_ss ? ssq_raw : 0.f;
        const float inv = a.qk_norm ? 1.0f / sqrtf(row16_sum(ssq) / (float)HD + a.eps) : 1.f;
        float q0[PPT], q1[PPT];
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const float y0 = x0[i] * inv * g0[i], y1 = x1[i] * inv * g1[i];
            q0[i] = live ? y0 * cs[i].x - y1 * cs[i].y : 0.f;
            q1[i] = live ? y0 * cs[i].y + y1 * cs[i].x : 0.f;
        }
        store_vec<PPT>(&Qs[qi][d0], q0);
        store_vec<PPT>(&Qs[qi][d0 + H2], q1);
    }
    // MULTI: this lane's query values for the score MFMAs into registers; then the shared space
    // takes the second stage's copies
    float4 qreg[MULTI ? DW / 16 : 1];
    if constexpr (MULTI) {
        lds_barrier();   // the query rows are in LDS
#pragma unroll
        for (int t = 0; t < DW / 16; ++t) qreg[t] = *(const float4*)&Qs[col][wave * DW + 16 * t + 4 * grp];
        lds_barrier();   // every wave has its query values
        issue_kv(K1, V1, wk0 + CK);
    }

    // the softmax and O are kept transposed: lane (col, grp) owns query vector col of the tile
    int lo_q, hi_q;
    {
        const int qv = qt * 16 + col;
        if (qv < a.NQ) row_range(a, qv / a.Hg, lo_q, hi_q);
        else { lo_q = 1; hi_q = 0; }
    }
    const float scale = 1.0f / sqrtf((float)HD);
    constexpr int NDT = DW / 16;
    floatx4 o[NDT];   // o[d][i] = O[q = col][wave * DW + 16 d + 4 grp + i]
#pragma unroll
    for (int d = 0; d < NDT; ++d) o[d] = (floatx4){0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    // score row m of a 16-key block is key 4 (m % 4) + m / 4 of the block, so lane (col, grp) gets
    // the keys 4 i + grp (i = 0..3): the keys its lane group feeds to PV step i
    const int krow = 4 * (col & 3) + (col >> 2);

    // one sub-chunk [c0, c0 + CK) from the stage (Kc, Vc); first: the sub-chunk whose first new rows
    // were loaded with the query
    auto sub_chunk = [&](int c0, TT (*Kc)[LDK], TT (*Vc)[LDV], bool first) __attribute__((always_inline)) {
        const int c1 = min(wk1, c0 + CK);
        // 2. this sub-chunk's K/V copies (and the loads before them) have landed in every wave. With
        //    MULTI the other stage's copies were issued after them and are the last NPW loads of the
        //    wave: a wave's loads land in order, so at most NPW left in flight means these are in.
        int p_lo, p_hi;
        new_rows(c0, p_lo, p_hi);
        if constexpr (MULTI) {
            wait_vmcnt<NPW>();
            lds_barrier();
        } else {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        // 3. own layers write the new rows, normalised and rotated, into the stage and the plane
        //    (the 16-thread groups are whole, so the row sums in store_row stay inside live groups)
        if (p_lo < p_hi) {
            if (!first && p_lo + ri < p_hi) load_row(p_lo + ri);
            if (p_lo + ri < p_hi) store_row(p_lo + ri, c0, Kc, Vc);
            for (int pr = p_lo + 16; pr < p_hi; pr += 16)
                if (pr + ri < p_hi) {
                    load_row(pr + ri);
                    store_row(pr + ri, c0, Kc, Vc);
                }
            // MULTI: the plane writes are complete inside this block, so the compiler needs no
            // wait where it joins the path without new rows for the registers they read (it would
            // otherwise wait for the next stage's copies on every sub-chunk); only sub-chunks with
            // new rows pay for it
            if constexpr (MULTI) wait_vmcnt<0>();
            lds_barrier();   // the new rows are in the stage
        }

        // 4. partial scores over this wave's dims, transposed (S^T = K Q^T): lane (col, grp) gets
        //    S[q = col][key 4 i + grp] of each 16-key block
        floatx4 sacc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[kb] = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < DW / 16; ++t) {
            const int d = wave * DW + 16 * t + 4 * grp;
            float4 qa;
            if constexpr (MULTI) qa = qreg[t];
            else qa = *(const float4*)&Qs[col][d];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                float4 kv4;
                if constexpr (KVB) {
                    const uint2 b = *(const uint2*)&Kc[kb * 16 + krow][d];
                    kv4.x = __builtin_bit_cast(float, b.x << 16);
                    kv4.y = __builtin_bit_cast(float, b.x & 0xffff0000u);
                    kv4.z = __builtin_bit_cast(float, b.y << 16);
                    kv4.w = __builtin_bit_cast(float, b.y & 0xffff0000u);
                } else {
                    kv4 = *(const float4*)&Kc[kb * 16 + krow][d];
                }
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv4.x, qa.x, sacc[kb], 0, 0, 0);
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv4.y, qa.y, sacc[kb], 0, 0, 0);
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv4.z, qa.z, sacc[kb], 0, 0, 0);
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv4.w, qa.w, sacc[kb], 0, 0, 0);
            }
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) *(floatx4*)&Sp[wave][col][kb * 16 + 4 * grp] = sacc[kb];
        lds_barrier();

        // 5. softmax update for the lane's vector over the sub-chunk (every wave for all 16
        //    vectors; the sums over the four waves' dims are taken in wave order). The maximum and
        //    the sum run over the lane's 4 KB keys, then over the four lane groups.
        float sv[KB][4];
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            floatx4 sp[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) sp[w] = *(const floatx4*)&Sp[w][col][kb * 16 + 4 * grp];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = c0 + kb * 16 + 4 * i + grp;
                const float sum = ((sp[0][i] + sp[1][i]) + sp[2][i]) + sp[3][i];
                sv[kb][i] = (key < c1 && key >= lo_q && key <= hi_q) ? sum * scale : -INFINITY;
                mx = fmaxf(mx, sv[kb][i]);
            }
        }
        mx = rows4_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sv[kb][i] = (sv[kb][i] == -INFINITY) ? 0.f : expf(sv[kb][i] - m_new);
                ps += sv[kb][i];
            }
        ps = rows4_sum(ps);
        l_run = l_run * alpha + ps;
        m_run = m_new;
#pragma unroll
        for (int d = 0; d < NDT; ++d) o[d] *= alpha;

        // 6. O^T += V^T P^T for this wave's dims: step (kb, i) takes the keys kb 16 + 4 i + grp,
        //    whose probabilities the lane holds
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int vr = kb * 16 + 4 * i + grp;
#pragma unroll
                for (int d = 0; d < NDT; ++d) {
                    float vb;
                    if constexpr (KVB) vb = bf16_to_f32(Vc[vr][wave * DW + 16 * d + col]);
                    else vb = Vc[vr][wave * DW + 16 * d + col];
                    o[d] = __builtin_amdgcn_mfma_f32_16x16x4f32(vb, sv[kb][i], o[d], 0, 0, 0);
                }
            }
    };
    if constexpr (MULTI) {
        // the sub-chunks alternate between the stages (the first two's copies went out above). Each
        // stage is refilled two sub-chunks ahead after a barrier (every wave has read it), also
        // past the last sub-chunk, so every stage read follows the same copies on every path; the
        // stages are named in each call, so the compiler sees that the copies in flight write the
        // other stage. The copies still in flight at the end are waited for before the exit.
        for (int c0 = wk0; c0 < wk1; c0 += 2 * CK) {
            sub_chunk(c0, K0, V0, false);
            lds_barrier();
            issue_kv(K0, V0, c0 + 2 * CK);
            if (c0 + CK < wk1) sub_chunk(c0 + CK, K1, V1, false);
            lds_barrier();
            issue_kv(K1, V1, c0 + 3 * CK);
        }
        wait_vmcnt<0>();
    } else if (wk0 < wk1) {
        sub_chunk(wk0, K0, V0, true);   // the only sub-chunk
    }

    // 7. this workgroup's partial: unnormalised O (each wave its dims), the running max and sum
    constexpr int PLD = attn_part_ld(HD);
    const size_t tile_base = ((size_t)qt * a.nkv + g) * a.n_chunks;
    float* part = a.part + (tile_base + chunk) * 16 * PLD + (size_t)col * PLD;
#pragma unroll
    for (int d = 0; d < NDT; ++d) *(floatx4*)&part[wave * DW + 16 * d + 4 * grp] = o[d];
    if (wave == 0 && grp == 0) {
        part[HD] = m_run;
        part[HD + 1] = l_run;
    }
}

// Merge of the chunks of one (q tile, KV head): one 256-thread block per (query vector, 64 dims).
// Wave w takes the chunks [w q, (w + 1) q), q = ceil(n_chunks / 4) <= QMAX: lane d loads its dim of
// every chunk, lane j the running maximum and sum of chunk w q + j, and every wave the maxima of all
// chunks (lane j those of chunks j + 64 u), all in one round of loads, so each wave has the overall
// maximum without an exchange. Chunk indices past the last chunk are clamped to it for the loads
// and masked after. The chunk weights are computed once per chunk (lane j) and broadcast from it.
// Every sum runs in a fixed order (within the 16-lane rows, across the rows, chunks in order, then
// the waves in order).
template <int HD, int QMAX>   // QMAX: chunks per wave at most (16, 32, or 64 for up to kAttnMaxChunks)
__global__ __launch_bounds__(256) void k_attn_combine(AttnK a) {
    static_assert(QMAX <= 64, "one lane per chunk of a wave");
    constexpr int NU = (4 * QMAX + 63) / 64;   // rounds of 64 chunk maxima
    __shared__ float denw[4], numw[4][64];
    const int dgroups = HD / 64;
    const int dg = blockIdx.x % dgroups;
    const int qvl = (blockIdx.x / dgroups) % 16;
    const int tile = blockIdx.x / (dgroups * 16);            // qt * nkv + g
    const int g = tile % a.nkv, qt = tile / a.nkv;
    const int qv = qt * 16 + qvl;
    if (qv >= a.NQ) return;   // uniform in the block
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nc = a.n_chunks;
    const int q = (nc + 3) / 4;
    constexpr int PLD = attn_part_ld(HD);
    const size_t cstride = (size_t)16 * PLD;
    const float* base = a.part + (size_t)tile * nc * cstride + (size_t)qvl * PLD;
    const int d = dg * 64 + lane;
    const int cw = wave * q;                              // this wave's first chunk
    const int nw = max(0, min(q, nc - cw));               // and its number of chunks
    float v[QMAX];
#pragma unroll
    for (int i = 0; i < QMAX; ++i) v[i] = base[(size_t)min(cw + i, nc - 1) * cstride + d];
    const float* pj = base + (size_t)min(cw + lane, nc - 1) * cstride + HD;
    const float mj_raw = pj[0], sj_raw = pj[1];
    float mu[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) mu[u] = base[(size_t)min(lane + 64 * u, nc - 1) * cstride + HD];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < NU; ++u)
        if (lane + 64 * u < nc) mx = fmaxf(mx, mu[u]);
    mx = wave64_max(mx);
    const bool lj = lane < nw;
    const float mj = lj ? mj_raw : -INFINITY;
    const float ej = mj == -INFINITY ? 0.f : expf(mj - mx);
    const float den = wave64_sum(lj ? ej * sj_raw : 0.f);
    float num = 0.f;
#pragma unroll
    for (int i = 0; i < QMAX; ++i)
        if (i < nw) num += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ej), i)) * v[i];
    numw[wave][lane] = num;
    if (lane == 0) denw[wave] = den;
    __syncthreads();
    if (wave == 0) {
        const float t = ((numw[0][lane] + numw[1][lane]) + numw[2][lane]) + numw[3][lane];
        const float dn = ((denw[0] + denw[1]) + denw[2]) + denw[3];
        const int mm = qv / a.Hg, h = g * a.Hg + qv % a.Hg;
        a.out[(size_t)mm * a.Hq * HD + (size_t)h * HD + d] = f32_to_bf16(t / dn);
    }
}

// ---------------------------------------------------------------------------------------------
// argmax (first index of the maximum, NaN never wins) and the greedy longest-prefix accept
// ([CARD], "How it is used"; [PR2236], the acceptance tool).
// ---------------------------------------------------------------------------------------------
constexpr int kArgmaxSpan = 4096;

__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
    // (v, i) beats (bv, bi) if v is a number and (bv is not, or v > bv, or v == bv and i < bi)
    if (v != v) return;
    if (bi < 0 || bv != bv || v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__global__ __launch_bounds__(256) void k_argmax_partial(const float* __restrict__ logits, int V, int nb,
                                                        float* __restrict__ pv, int* __restrict__ pi) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int b = blockIdx.x, row = blockIdx.y;
    const int lo = b * kArgmaxSpan, hi = min(V, lo + kArgmaxSpan);
    const float* lr = logits + (size_t)row * V;
    float bv = 0.f;
    int bi = -1;
    // the span's 16 values per thread are loaded in one round (four 16-byte loads, coalesced over
    // the block) before any comparison; "better" is a total order, so the visiting order does not
    // change the result. A span that ends early or an unaligned row takes the scalar path.
    constexpr int kVec = kArgmaxSpan / 1024;   // 16-byte loads per thread
    const bool vec_ok = ((V & 3) == 0) && (((uintptr_t)lr & 15) == 0);
    float4 v4[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        const int i0 = lo + j * 1024 + (int)threadIdx.x * 4;
        if (vec_ok && i0 + 3 < hi) v4[j] = *(const float4*)(lr + i0);
    }
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        const int i0 = lo + j * 1024 + (int)threadIdx.x * 4;
        if (vec_ok && i0 + 3 < hi) {
            better(bv, bi, v4[j].x, i0);
            better(bv, bi, v4[j].y, i0 + 1);
            better(bv, bi, v4[j].z, i0 + 2);
            better(bv, bi, v4[j].w, i0 + 3);
        } else {
            for (int e = 0; e < 4; ++e)
                if (i0 + e < hi) better(bv, bi, lr[i0 + e], i0 + e);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (oi >= 0) better(bv, bi, ov, oi);
    }
    if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        bv = sv[0];
        bi = si[0];
        for (int w = 1; w < 4; ++w) if (si[w] >= 0) better(bv, bi, sv[w], si[w]);
        pv[(size_t)row * nb + b] = bv;
        pi[(size_t)row * nb + b] = bi;
    }
}

// ---------------------------------------------------------------------------------------------
// Sampled rows (temperature T > 0; [CARD] "How it is used": every position is sampled and compared
// with the draft). Row i's draw is the first index of the maximum of the Gumbel-perturbed scores
// fmaf(z_ij, 1/T, -log(-log u_ij)), which follows softmax(z_i / T). u_ij = ((x >> 9) + 1/2) / 2^23
// with x the word j % 4 of one Philox4x32-10 block (Salmon, Moraes, Dror, Shaw, SC 2011) at counter
// (j / 4, i, offset low, offset high) under key (seed low, seed high); every such u is exact in fp32
// and lies in [2^-24, 1 - 2^-24], so the noise is finite. Each thread draws four consecutive entries
// from one block and reads them with one 16-byte load.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {   // the key takes a Weyl step before every round after the first
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
        const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    }
    return c;
}

__global__ __launch_bounds__(256) void k_sample_partial(const float* __restrict__ logits, int V, int nb,
                                                        float* __restrict__ pv, int* __restrict__ pi, SampleArgs sa) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int b = blockIdx.x, row = blockIdx.y;
    const int lo = b * kArgmaxSpan, hi = min(V, lo + kArgmaxSpan);   // lo is a multiple of 4
    const float* lr = logits + (size_t)row * V;
    float bv = 0.f;
    int bi = -1;
    for (int q = (lo >> 2) + (int)threadIdx.x; 4 * q < hi; q += 256) {
        const uint4 x = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)row, sa.off0, sa.off1), sa.key0, sa.key1);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
        float z[4];
        const int j0 = 4 * q;
        if (j0 + 4 <= hi && (V & 3) == 0) {
            const float4 v = *(const float4*)(lr + j0);
            z[0] = v.x; z[1] = v.y; z[2] = v.z; z[3] = v.w;
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) z[w] = j0 + w < hi ? lr[j0 + w] : 0.f;
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (j0 + w >= hi) break;
            const float u = ((float)(xs[w] >> 9) + 0.5f) * (1.0f / 8388608.0f);
            const float g = -logf(-logf(u));
            better(bv, bi, __builtin_fmaf(z[w], sa.inv_t, g), j0 + w);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (oi >= 0) better(bv, bi, ov, oi);
    }
    if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        bv = sv[0];
        bi = si[0];
        for (int w = 1; w < 4; ++w) if (si[w] >= 0) better(bv, bi, sv[w], si[w]);
        pv[(size_t)row * nb + b] = bv;
        pi[(size_t)row * nb + b] = bi;
    }
}

// One wave per row (64 x k threads): every row's partials are loaded in the same round.
__global__ __launch_bounds__(64 * kMaxRows) void k_accept(const float* __restrict__ pv, const int* __restrict__ pi, int nb,
                                                          int k, const int32_t* __restrict__ tokens,
                                                          int32_t* __restrict__ out_tokens, int32_t* __restrict__ n_acc,
                                                          int32_t* __restrict__ argmax_out) {
    __shared__ int y[kMaxRows];
    const int lane = threadIdx.x & 63;
    const int row = threadIdx.x >> 6;
    if (row < k) {
        float bv = 0.f;
        int bi = -1;
        for (int b = lane; b < nb; b += 64) {
            const int i = pi[(size_t)row * nb + b];
            const float v = pv[(size_t)row * nb + b];
            if (i >= 0) better(bv, bi, v, i);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (oi >= 0) better(bv, bi, ov, oi);
        }
        if (lane == 0) y[row] = bi < 0 ? 0 : bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        if (argmax_out) for (int r = 0; r < k; ++r) argmax_out[r] = y[r];
        if (tokens) {
            int acc = 0;
            while (acc < k - 1 && tokens[acc + 1] == y[acc]) ++acc;
            for (int i = 0; i < acc; ++i) out_tokens[i] = tokens[i + 1];
            out_tokens[acc] = y[acc];
            n_acc[0] = acc;
        }
    }
}

__global__ void k_steer(float* logits, int k, int V, const int32_t* tok, const float* add) {
    const int i = threadIdx.x;
    if (i < k) {
        const int t = tok[i];
        if (t >= 0 && t < V) logits[(size_t)i * V + t] += add[i];
    }
}

}  // namespace

hipError_t launch_repack_q4_1(const uint8_t* canon, int n_out, int n_in, uint8_t* codes, uint8_t* sm, int G, int col0,
                              int gu_mode, hipStream_t st) {
    const int nb = n_in / 32;
    const size_t n = (size_t)n_out * nb;
    hipLaunchKernelGGL(k_repack, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, canon, n_out, nb, codes, sm, G,
                       col0, gu_mode);
    return hipGetLastError();
}

hipError_t launch_dequant_q4_1(const WMat& w, int tile0, int gu, int n_out, float* out, hipStream_t st) {
    const size_t n = (size_t)n_out * w.K;
    hipLaunchKernelGGL(k_dequant, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, w.codes, w.sm, w.G, tile0, gu,
                       n_out, w.K, out);
    return hipGetLastError();
}

hipError_t launch_rope_table(float2* table, int max_ctx, int hd, double base, hipStream_t st) {
    const size_t n = (size_t)max_ctx * (hd / 2);
    hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, table, max_ctx, hd, base);
    return hipGetLastError();
}

hipError_t launch_embed(const int32_t* tokens, int fill_token, int rows, const uint16_t* embed, int V, int H,
                        float scale, float* x, float* ss, hipStream_t st) {
    hipLaunchKernelGGL(k_embed, dim3((H + 255) / 256, rows), dim3(256), 0, st, tokens, fill_token, embed, V, H, scale,
                       x, ss);
    return hipGetLastError();
}

hipError_t launch_sumsq(const float* x, int ldx, int rows, int H, float* ss, hipStream_t st) {
    hipLaunchKernelGGL(k_sumsq, dim3((H + 255) / 256, rows), dim3(256), 0, st, x, ldx, H, ss);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, int ldx, int rows, int H, const uint16_t* g, float eps, uint16_t* out, int ldo,
                          hipStream_t st) {
    hipLaunchKernelGGL(k_rmsnorm, dim3(rows), dim3(256), 0, st, x, ldx, H, g, eps, out, ldo);
    return hipGetLastError();
}

hipError_t launch_rope_append(const RopeAppend& a, hipStream_t st) {
    const int rows = a.rows > a.rows_q ? a.rows : a.rows_q;
    hipLaunchKernelGGL(k_rope_append, dim3(rows, a.Hq + a.nkv), dim3(64), 0, st, a);
    return hipGetLastError();
}

namespace {
AttnK make_attn(const Attn& x) {
    AttnK a{};
    a.qkv = x.qkv;
    a.ss = x.ss;
    a.ldq = x.ldq;
    a.q_norm = x.q_norm;
    a.k_norm = x.k_norm;
    a.qk_norm = x.qk_norm;
    a.eps = x.eps;
    a.rope = x.rope;
    a.plane = x.plane;
    a.kv_bf16 = x.kv_bf16;
    a.ring_cap = x.ring_cap;
    a.w = x.w;
    a.own = x.own;
    a.M = x.M;
    a.Hq = x.Hq;
    a.nkv = x.nkv;
    a.Hg = x.Hq / x.nkv;
    a.NQ = x.M * a.Hg;
    a.n_qt = (a.NQ + 15) / 16;
    a.causal = x.causal;
    a.pos0 = x.pos0;
    a.window = x.window;
    a.ctx_lo = x.ctx_lo;
    a.ctx_hi = x.ctx_hi;
    a.np0 = x.np0;
    a.np1 = x.np1;
    a.sp = x.sp;
    a.r_lo = x.r_lo;
    a.r_hi = x.r_hi;
    int lo, hi;
    if (x.causal) {
        hi = x.pos0 + x.M - 1;
        lo = (x.window > 0 && x.pos0 - x.window + 1 > 0) ? x.pos0 - x.window + 1 : 0;
    } else {
        lo = x.ctx_lo;
        hi = x.ctx_hi;
    }
    // the new rows must lie inside the key range (they are appended by the chunk that holds them)
    if (x.own && x.np1 > x.np0) {
        lo = std::min(lo, x.np0);
        hi = std::max(hi, x.np1 - 1);
    }
    a.key_lo = lo;
    a.n_keys = hi - lo + 1;
    a.dpos = x.dpos;
    a.n_ctx = x.n_ctx;
    // the plan covers the keys of rows at pos_plan when given (a bound shared by passes at lower
    // positions: a later pass there leaves trailing chunks empty)
    int plan_keys = a.n_keys;
    if (x.causal && x.pos_plan > x.pos0) {
        const int plo = (x.window > 0 && x.pos_plan - x.window + 1 > 0) ? x.pos_plan - x.window + 1 : 0;
        plan_keys = std::max(plan_keys, x.pos_plan + x.M - plo);
    }
    // One sub-chunk per workgroup while that takes at most kAttnMaxChunks chunks and 768
    // workgroups. Longer key ranges: workgroups of spw sub-chunks, planned to run in a single round
    // of as many workgroups per compute unit as the LDS holds, at most two (the kernel's 164-216
    // VGPRs leave two waves per SIMD; one workgroup's copies are in flight while another computes).
    const int tiles = a.n_qt * a.nkv;
    const int ck = attn_ck(x.hd);
    const int subs = (plan_keys + ck - 1) / ck;
    if (subs <= kAttnMaxChunks && (long)subs * tiles <= 768) {
        a.spw = 1;
        a.n_chunks = subs;
    } else {
        const int per_cu = std::max(1, std::min(2, (int)(kLdsPerCu / attn_lds_bytes(x.hd, x.kv_bf16 != 0, true))));
        const int nch = std::max(1, std::min(kAttnMaxChunks, per_cu * x.n_cu / tiles));
        a.spw = (subs + nch - 1) / nch;
        a.n_chunks = (subs + a.spw - 1) / a.spw;
    }
    a.part = x.part;
    a.counters = x.counters;
    a.out = x.out;
    return a;
}
}  // namespace

size_t attn_part_floats_needed(const Attn& x) {
    const AttnK a = make_attn(x);
    return (size_t)a.n_qt * a.nkv * a.n_chunks * 16 * attn_part_ld(x.hd);
}

int64_t attn_plan_key(const Attn& x) {
    const AttnK a = make_attn(x);
    return (int64_t)a.n_chunks * 65536 + a.spw;
}

namespace {
template <int HD>
void launch_attn(const AttnK& a, int grid, int cgrid, hipStream_t st) {
    if (a.spw > 1) {
        if (a.kv_bf16) hipLaunchKernelGGL((k_attention<HD, true, true>), dim3(grid), dim3(256), 0, st, a);
        else hipLaunchKernelGGL((k_attention<HD, false, true>), dim3(grid), dim3(256), 0, st, a);
    } else {
        if (a.kv_bf16) hipLaunchKernelGGL((k_attention<HD, true, false>), dim3(grid), dim3(256), 0, st, a);
        else hipLaunchKernelGGL((k_attention<HD, false, false>), dim3(grid), dim3(256), 0, st, a);
    }
    static_assert(kAttnMaxChunks <= 4 * 64, "the combine's wider form takes 64 chunks per wave");
    // chunks per wave of the combine: the smallest form that holds them (every form issues QMAX loads)
    if (a.n_chunks <= 64) hipLaunchKernelGGL((k_attn_combine<HD, 16>), dim3(cgrid), dim3(256), 0, st, a);
    else if (a.n_chunks <= 128) hipLaunchKernelGGL((k_attn_combine<HD, 32>), dim3(cgrid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_attn_combine<HD, 64>), dim3(cgrid), dim3(256), 0, st, a);
}
}  // namespace

hipError_t launch_attention(const Attn& x, hipStream_t st) {
    const AttnK a = make_attn(x);
    if (attn_part_floats_needed(x) > x.part_floats || a.n_qt * a.nkv > x.n_counters) return hipErrorInvalidValue;
    if (a.n_chunks > kAttnMaxChunks) return hipErrorInvalidValue;
    if (a.ring_cap > 0 && a.ring_cap < 4) return hipErrorInvalidValue;   // the copies step slots by 4
    const int grid = (a.n_chunks * a.nkv + 7) / 8 * 8 * a.n_qt;
    const int cgrid = a.n_qt * a.nkv * 16 * (x.hd / 64);
    switch (x.hd) {
        case 64: launch_attn<64>(a, grid, cgrid, st); break;
        case 128: launch_attn<128>(a, grid, cgrid, st); break;
        case 256: launch_attn<256>(a, grid, cgrid, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int argmax_blocks(int V) { return (V + kArgmaxSpan - 1) / kArgmaxSpan; }

hipError_t launch_argmax_accept(const float* logits, int k, int V, const int32_t* tokens, float* part_val, int* part_idx,
                                int nb, int32_t* out_tokens, int32_t* n_acc, int32_t* argmax_out, hipStream_t st,
                                const SampleArgs* sample) {
    if (k < 1 || k > kMaxRows) return hipErrorInvalidValue;
    if (sample)
        hipLaunchKernelGGL(k_sample_partial, dim3(nb, k), dim3(256), 0, st, logits, V, nb, part_val, part_idx, *sample);
    else
        hipLaunchKernelGGL(k_argmax_partial, dim3(nb, k), dim3(256), 0, st, logits, V, nb, part_val, part_idx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_accept, dim3(1), dim3(64 * k), 0, st, part_val, part_idx, nb, k, tokens, out_tokens, n_acc,
                       argmax_out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Argmax partials of the allocation-free greedy accept: one file-scope device array per GPU,
// [kMaxRows][kStaticAcceptBlocks] values then as many indices. Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device address): each device's
// address comes from hipGetSymbolAddress, taken once per device with that device current.
// ---------------------------------------------------------------------------------------------
__device__ __align__(256) uint8_t scratch[kStaticAcceptScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_accept_scratch(int device, float** part_val, int** part_idx) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device) return hipErrorInvalidDevice;   // the caller makes the device current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *part_val = (float*)g_scratch_ptr[device];
    *part_idx = (int*)((uint8_t*)g_scratch_ptr[device] + (size_t)kMaxRows * kStaticAcceptBlocks * sizeof(float));
    return hipSuccess;
}

hipError_t launch_set_i64(int64_t* dst, int64_t v, hipStream_t st) {
    hipLaunchKernelGGL(k_set_i64, dim3(1), dim3(1), 0, st, dst, v);
    return hipGetLastError();
}

hipError_t launch_steer(float* logits, int k, int V, const int32_t* tok, const float* add, hipStream_t st) {
    hipLaunchKernelGGL(k_steer, dim3(1), dim3(64), 0, st, logits, k, V, tok, add);
    return hipGetLastError();
}

}  // namespace bvf
