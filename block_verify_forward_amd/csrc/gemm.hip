// Small-M (k <= 16 rows) weight-streaming GEMM for gfx950, Q4_1 or bf16 weights.
//
// The verify pass is a skinny GEMM over the whole weight image: k <= 16 activation rows against
// every weight column ([PR2303] "What changes": all k drafted rows go through every layer in one
// pass over the weights). Each weight byte is read from HBM once per launch; the k rows share it.
// The contraction is real (M = k), so it runs on the bf16 MFMA v_mfma_f32_16x16x32_bf16 with the
// k rows padded to the 16-row tile.
//
// Q4_1 ([CARD], "Weights" row): weight = scale * code + min over 32-weight blocks. The dequant is
// factored and exact: the code q is placed in a bf16 as 0x4180 | q << 3 = 16 + q (exact: at 16 the
// bf16 step is 1/8), one MFMA per 32-weight block gives C' = sum_k x_k (16 + q_k), a second MFMA
// against ones gives the block sum S = sum_k x_k, and the block contributes
// scale * C' + (min - 16 scale) * S, i.e. exactly sum_k x_k (scale q_k + min). Products bf16 x bf16
// are exact in fp32; accumulation is fp32. The offset 16 (not 128) keeps the cancellation small.
//
// Work split: an item = one wave = NT column tiles (16 columns each) over a K range of
// superblocks (128 K); items of one column group are consecutive and split K when the matrix has
// few columns. Split-K partials are summed in a fixed order by the last wave to arrive (integer
// arrival counter), so results are deterministic. Workgroup ids are remapped so consecutive
// logical workgroups share an XCD (the hardware deals workgroups round-robin over the 8 XCDs).
#include "bvf_impl.hpp"

namespace bvf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct KArgs {
    const uint8_t* codes;
    const uint8_t* sm;
    int G, K;
    int tile0, tile_stride;
    const uint16_t* A;
    int lda, M;
    float* y;
    int ldy;
    uint16_t* out;
    int ldo;
    uint16_t* taps;
    int ldt;
    float* partial;
    int* counters;
    int S, sb_per_split, n_groups, n_cols;
    int half;   // STORE on a gate|up image: -1 all 16 columns, 0 the gate half, 1 the up half
    // RMSNorm folded into the staging of A (xsrc != nullptr): A = bf16(x * rinv * gain) with
    // rinv = 1 / sqrt(sum(ss_in[m][0 .. n_ss)) / K + eps)
    const float* xsrc;
    int ldx;
    const float* ss_in;
    int n_ss;
    const uint16_t* gain;
    float eps;
    float* ss_out;   // STORE / RESID: per row and 16-column tile, the sum of squares of the outputs
};

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float half_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Logical workgroup id: consecutive ids live on the same XCD.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int q = n >> 3, r = n & 7, x = b & 7, i = b >> 3;
    return x * q + (x < r ? x : r) + i;
}

template <int FMT, int NT>
struct Frag;

template <int NT>
struct Frag<W_Q4_1, NT> {
    u32x4 cw[NT];
    u32x4 sm[NT];
};

template <int NT>
struct Frag<W_BF16, NT> {
    u32x4 bw[NT][4];
};

// Weight bytes of superblock g for this lane (the only loads of the main loop).
template <int FMT, int NT>
__device__ __forceinline__ void load_frag(Frag<FMT, NT>& f, const KArgs& a, const int (&T)[NT], int g, int lane) {
    const int c = lane & 15, sub = lane >> 4;
    if constexpr (FMT == W_Q4_1) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const size_t base = (size_t)T[t] * a.G + g;
            f.cw[t] = __builtin_nontemporal_load((const u32x4*)a.codes + base * 64 + lane);
            f.sm[t] = __builtin_nontemporal_load((const u32x4*)a.sm + base * 16 + c);
        }
    } else {
        const uint16_t* W = (const uint16_t*)a.codes;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint16_t* row = W + (size_t)(T[t] * kTile + c) * a.K + (size_t)g * kSuper + sub * 8;
#pragma unroll
            for (int j = 0; j < 4; ++j) f.bw[t][j] = __builtin_nontemporal_load((const u32x4*)(row + j * 32));
        }
    }
}

// One superblock: A (this lane's row, 4 blocks of 8 bf16) comes from the LDS copy of the rows.
template <int FMT, int NT>
__device__ __forceinline__ void compute_frag(const Frag<FMT, NT>& f, const uint16_t* As_row, bool a_live,
                                             floatx4 (&acc)[NT]) {
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    const u32x4 z = {0u, 0u, 0u, 0u};
    u32x4 av4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) av4[j] = a_live ? *(const u32x4*)(As_row + j * 32) : z;
    if constexpr (FMT == W_Q4_1) {
        // Block j's two MFMAs are issued before block j-1's scale/min FMAs, so the MFMA latency is
        // covered while at most two blocks of results are live (sched barriers stop the scheduler
        // from hoisting every MFMA of the pipeline, which costs registers and occupancy).
        const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
        floatx4 bs[2], cc[2][NT];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            if (j < 4) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, av4[j]);
                bs[j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, ones), zero, 0, 0, 0);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const uint32_t w = f.cw[t][j];
                    const uint32_t M4 = 0x00780078u, O = 0x41804180u;   // nibble -> mantissa bits 3..6
                    const u32x4 b = {((w << 3) & M4) | O, ((w >> 1) & M4) | O, ((w >> 5) & M4) | O, ((w >> 9) & M4) | O};
                    cc[j & 1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, b), zero, 0, 0, 0);
                }
            }
            if (j > 0) {
                const int jp = j - 1;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const uint32_t smv = f.sm[t][jp];
                    const float s = half_lo(smv), mn = half_hi(smv);
                    const float mp = fmaf(-16.f, s, mn);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(s, cc[jp & 1][t][r], fmaf(mp, bs[jp & 1][r], acc[t][r]));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 av = __builtin_bit_cast(bf16x8, av4[j]);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, f.bw[t][j]), acc[t], 0, 0, 0);
        }
    }
}

template <int EPI, int NT>
__device__ __forceinline__ void epilogue(const KArgs& a, const floatx4 (&acc)[NT], int group, int lane) {
    const int c = lane & 15, sub = lane >> 4;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = (group * NT + t) * kTile + c;
        if constexpr (EPI == EPI_SWIGLU) {
            // a gate|up tile holds gate columns in lanes c < 8 and the matching up columns in c + 8
            floatx4 up;
#pragma unroll
            for (int r = 0; r < 4; ++r) up[r] = __shfl_xor(acc[t][r], 8);
            if (c < 8) {
                const int nh = (group * NT + t) * 8 + c;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 4 * sub + r;
                    if (m >= a.M) continue;
                    const float g = acc[t][r];
                    a.out[(size_t)m * a.ldo + nh] = f32_to_bf16(g / (1.0f + expf(-g)) * up[r]);
                }
            }
            continue;
        }
        float vout[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * sub + r;
            vout[r] = 0.f;
            if (m >= a.M) continue;
            if constexpr (EPI == EPI_STORE) {
                vout[r] = acc[t][r];
                if (a.half < 0) {
                    a.y[(size_t)m * a.ldy + n] = acc[t][r];
                } else if ((c >> 3) == a.half) {
                    a.y[(size_t)m * a.ldy + (group * NT + t) * 8 + (c & 7)] = acc[t][r];
                }
            } else {
                const float v = a.y[(size_t)m * a.ldy + n] + acc[t][r];
                vout[r] = v;
                a.y[(size_t)m * a.ldy + n] = v;
                if (a.taps) a.taps[(size_t)m * a.ldt + n] = f32_to_bf16(v);
            }
        }
        if (a.ss_out) {
            // per row, the sum of squares over this tile's 16 columns (lanes c = 0..15 of a row group)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float q = vout[r] * vout[r];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) q += __shfl_xor(q, o);
                const int m = 4 * sub + r;
                if (c == 0 && m < a.M) a.ss_out[(size_t)m * (a.n_cols / kTile) + group * NT + t] = q;
            }
        }
    }
}

// A workgroup = 4 waves = 4 column groups that share one K range (split). The workgroup copies
// its K range of the M activation rows into LDS once; each wave then streams only weight bytes,
// DEPTH superblocks ahead. At least 4 waves per SIMD (<= 128 registers) keep enough loads in
// flight to cover HBM latency.
template <int FMT, int EPI, int NT, int DEPTH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_gemm(KArgs a) {
    extern __shared__ uint16_t As[];   // [M][lds_ld] bf16, lds_ld = sb_per_split * 128 + 8
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: loop control stays scalar
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int quad = wg / a.S;
    const int split = wg - quad * a.S;
    const int group = quad * 4 + wave;
    if (quad * 4 >= a.n_groups) return;      // grid padding (whole workgroup, before any barrier)
    const bool live = group < a.n_groups;
    const int g0 = split * a.sb_per_split;
    const int g1 = min(a.G, g0 + a.sb_per_split);
    const int nsb = g1 - g0;
    const int lds_ld = a.sb_per_split * kSuper + 8;

    int T[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) T[t] = a.tile0 + ((live ? group : 0) * NT + t) * a.tile_stride;

    // weight prefetch first, then the activation rows into LDS
    Frag<FMT, NT> f[DEPTH];
    if (live) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
            if (d < nsb) load_frag<FMT, NT>(f[d], a, T, g0 + d, lane);
    }
    if (a.xsrc) {
        // RMSNorm of the rows: rinv from the producer's per-tile sums of squares, then the scaled
        // bf16 rows of this K range into LDS
        __shared__ float rinv_s[kMaxRows];
        for (int m = wave; m < a.M; m += 4) {
            float ssum = 0.f;
            for (int i = lane; i < a.n_ss; i += 64) ssum += a.ss_in[(size_t)m * a.n_ss + i];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) ssum += __shfl_xor(ssum, o);
            if (lane == 0) rinv_s[m] = 1.0f / sqrtf(ssum / (float)a.K + a.eps);
        }
        __syncthreads();
        const int per_row = nsb * (kSuper / 8);   // 8-element pieces per row
        for (int idx = threadIdx.x; idx < a.M * per_row; idx += 256) {
            const int m = idx / per_row, c8 = idx - m * per_row;
            const int k0 = g0 * kSuper + c8 * 8;
            const float4 x0 = *(const float4*)(a.xsrc + (size_t)m * a.ldx + k0);
            const float4 x1 = *(const float4*)(a.xsrc + (size_t)m * a.ldx + k0 + 4);
            const u32x4 gv = *(const u32x4*)(a.gain + k0);
            const float r = rinv_s[m];
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float g_lo = __builtin_bit_cast(float, gv[q] << 16);
                const float g_hi = __builtin_bit_cast(float, gv[q] & 0xffff0000u);
                o[q] = (uint32_t)f32_to_bf16(xs[2 * q] * r * g_lo) | ((uint32_t)f32_to_bf16(xs[2 * q + 1] * r * g_hi) << 16);
            }
            *(u32x4*)(As + m * lds_ld + c8 * 8) = o;
        }
    } else {
        const int per_row = nsb * (kSuper / 8);   // 16-byte pieces per row
        for (int idx = threadIdx.x; idx < a.M * per_row; idx += 256) {
            const int m = idx / per_row, c16 = idx - m * per_row;
            *(u32x4*)(As + m * lds_ld + c16 * 8) =
                *(const u32x4*)(a.A + (size_t)m * a.lda + (size_t)g0 * kSuper + c16 * 8);
        }
    }
    __syncthreads();
    if (!live) return;

    const int m_a = lane & 15, sub = lane >> 4;
    const bool a_live = m_a < a.M;
    const uint16_t* As_row = As + (a_live ? m_a : 0) * lds_ld + sub * 8;

    floatx4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = (floatx4){0.f, 0.f, 0.f, 0.f};

    int i = 0;
    for (; i + 2 * DEPTH <= nsb; i += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            compute_frag<FMT, NT>(f[d], As_row + (i + d) * kSuper, a_live, acc);
            load_frag<FMT, NT>(f[d], a, T, g0 + i + d + DEPTH, lane);
        }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        if (i + d < nsb) {
            compute_frag<FMT, NT>(f[d], As_row + (i + d) * kSuper, a_live, acc);
            if (i + d + DEPTH < nsb) load_frag<FMT, NT>(f[d], a, T, g0 + i + d + DEPTH, lane);
        }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (i + DEPTH + d < nsb) compute_frag<FMT, NT>(f[d], As_row + (i + DEPTH + d) * kSuper, a_live, acc);

    if (a.S > 1) {
        // Split-K hand-off without cache flushes: partials are stored at device scope (sc1), the
        // wave waits until its stores are performed, then bumps the group's arrival counter; the
        // last wave to arrive reads the partials at device scope and sums them in split order.
        const int c = lane & 15;
        float* P = a.partial + (size_t)split * a.M * a.n_cols;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int n = (group * NT + t) * kTile + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * sub + r;
                if (m < a.M) __hip_atomic_store(P + (size_t)m * a.n_cols + n, acc[t][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        int old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(&a.counters[group], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0);
        if (old != a.S - 1) return;
        // sum the splits in order; the device-scope loads are issued eight at a time
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int n = (group * NT + t) * kTile + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * sub + r;
                const int mm = m < a.M ? m : 0;
                const float* src = a.partial + (size_t)mm * a.n_cols + n;
                const size_t stride = (size_t)a.M * a.n_cols;
                float s = 0.f;
                for (int sp0 = 0; sp0 < a.S; sp0 += 8) {
                    float v[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        v[i] = (sp0 + i < a.S && sp0 + i != split)
                                   ? __hip_atomic_load(src + (size_t)(sp0 + i) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                   : 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (sp0 + i < a.S) s += (sp0 + i == split) ? acc[t][r] : v[i];
                }
                acc[t][r] = s;
            }
        }
        if (lane == 0) __hip_atomic_store(&a.counters[group], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    epilogue<EPI, NT>(a, acc, group, lane);
}

// One 16-column tile per wave; the pipeline is 3 (Q4_1: 8 weight registers per stage) or 2 (bf16:
// 16 per stage) superblocks deep, which fits 128 registers without spills.
template <int FMT, int EPI>
hipError_t launch_nt(int NT, const KArgs& k, int grid, size_t lds, hipStream_t st) {
    if (NT != 1) return hipErrorInvalidValue;
    constexpr int D = FMT == W_Q4_1 ? 3 : 2;
    hipLaunchKernelGGL((k_gemm<FMT, EPI, 1, D>), dim3(grid), dim3(256), lds, st, k);
    return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(const GemmLaunch& L) {
    GemmPlan p{};
    const int tiles = L.n_run_tiles, G = L.w.G;
    const int NT = 1;
    const int groups = tiles / NT;
    const int quads = (groups + 3) / 4;
    // LDS holds the workgroup's K range of the M rows: bounds the superblocks per split
    const size_t budget = L.fmt == W_Q4_1 ? kLdsBudgetQ4 : kLdsBudgetBf16;
    int sb_max = (int)((budget / (2 * (size_t)L.M) - 8) / kSuper);
    if (sb_max < 1) sb_max = 1;
    int S = L.S;
    if (S == 0) {
        const int target_waves = 2048;
        S = (target_waves + groups - 1) / groups;
        if (S > G) S = G;
        if (S < 1) S = 1;
    }
    int sb = (G + S - 1) / S;
    if (sb > sb_max) sb = sb_max;
    S = (G + sb - 1) / sb;
    if (S > 1 && ((size_t)S * L.M * tiles * kTile > L.partial_floats || groups > L.n_counters)) S = -1;  // no fit
    p.NT = NT;
    p.S = S;
    p.sb_per_split = sb;
    p.n_groups = groups;
    p.items = groups * (S > 0 ? S : 0);
    // The grid is a multiple of 8 * S, so each XCD's contiguous range of logical workgroup ids holds
    // whole column groups: all splits of a group run on one XCD (one L2).
    p.grid = quads * (S > 0 ? S : 0);
    if (S > 1) {
        const int unit = 8 * S;
        p.grid = (p.grid + unit - 1) / unit * unit;
    }
    p.lds = (size_t)L.M * (sb * kSuper + 8) * 2;
    return p;
}

hipError_t launch_gemm(const GemmLaunch& L, hipStream_t st) {
    if (L.M < 1 || L.M > kMaxRows) return hipErrorInvalidValue;
    const GemmPlan p = plan_gemm(L);
    if (p.S < 1 || L.n_run_tiles % p.NT != 0) return hipErrorInvalidValue;
    KArgs k;
    k.codes = L.w.codes;
    k.sm = L.w.sm;
    k.G = L.w.G;
    k.K = L.w.K;
    k.tile0 = L.tile0;
    k.tile_stride = L.tile_stride;
    k.A = L.A;
    k.lda = L.lda;
    k.M = L.M;
    k.y = L.y;
    k.ldy = L.ldy;
    k.out = L.out;
    k.ldo = L.ldo;
    k.taps = L.taps;
    k.ldt = L.ldt;
    k.partial = L.partial;
    k.counters = L.counters;
    k.S = p.S;
    k.sb_per_split = p.sb_per_split;
    k.n_groups = p.n_groups;
    k.n_cols = L.n_run_tiles * kTile;
    k.half = L.half;
    k.xsrc = L.xsrc;
    k.ldx = L.ldx;
    k.ss_in = L.ss_in;
    k.n_ss = L.n_ss;
    k.gain = L.gain;
    k.eps = L.eps;
    k.ss_out = L.ss_out;
    if (L.fmt == W_Q4_1) {
        switch (L.epi) {
            case EPI_STORE: return launch_nt<W_Q4_1, EPI_STORE>(p.NT, k, p.grid, p.lds, st);
            case EPI_RESID: return launch_nt<W_Q4_1, EPI_RESID>(p.NT, k, p.grid, p.lds, st);
            case EPI_SWIGLU: return launch_nt<W_Q4_1, EPI_SWIGLU>(p.NT, k, p.grid, p.lds, st);
        }
    } else if (L.epi == EPI_STORE) {
        return launch_nt<W_BF16, EPI_STORE>(p.NT, k, p.grid, p.lds, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace bvf
