// Small-M (k <= 16 rows; up to 64 rows for prefill chunks) weight-streaming GEMM for gfx950, Q4_1
// or bf16 weights.
//
// The verify pass is a skinny GEMM over the whole weight image: k <= 16 activation rows against
// every weight column ([PR2303] "What changes": all k drafted rows go through every layer in one
// pass over the weights). Each weight byte is read from HBM once per launch; the k rows share it.
// The contraction is real (M = k), so it runs on the bf16 MFMA v_mfma_f32_16x16x32_bf16 with the
// k rows padded to the 16-row tile.
//
// Q4_1 ([CARD], "Weights" row): weight = scale * code + min over 32-weight blocks. The dequant is
// factored and exact: the code q is placed in a bf16 as 0x4180 | q << 3 = 16 + q (exact: at 16 the
// bf16 step is 1/8), one MFMA per 32-weight block gives C' = sum_k x_k (16 + q_k), and the block
// contributes scale * C' + (min - 16 scale) * S with S = sum_k x_k, i.e. exactly
// sum_k x_k (scale q_k + min). The S terms of the four blocks of a superblock are one fp32 MFMA
// 16x16x4 (rows x blocks times blocks x columns) from block sums computed once per workgroup.
// Products bf16 x bf16 are exact in fp32; accumulation is fp32. The offset 16 (not 128) keeps the
// cancellation small.
//
// Weight streaming: every wave owns a ring of R superblock slots in LDS, filled by direct
// global->LDS loads (global_load_lds_dwordx4), R superblocks ahead of the MFMAs. The ring holds no
// loop-carried registers, so the loads stay in flight across loop iterations; the wave waits with
// s_waitcnt vmcnt for exactly the slot it consumes next (vector-memory loads complete in order).
//
// Work split: an item = one 16-column tile over one K range (split). A workgroup = 4 waves that
// share one split; it stages the M activation rows of that K range in LDS once (RMSNorm folded in
// when requested), then each wave streams its items (tiles wv, wv + WV, ...) through its ring.
// Split-K partials are summed in a fixed order by the last wave to arrive (integer arrival
// counter), so results are deterministic.
//
// Wider chunks (prefill, [PR2303] "Proof": the chunk arms of the state test): with M up to 64 rows
// a wave's dequantised superblock feeds MT = 2 or 4 row tiles of 16 (one MFMA per tile and block),
// so the weight stream and the dequantisation are paid once for all rows and the matrix cores take
// the extra work. Such workgroups run at most 8 waves (two per SIMD, for the MT accumulators). Their
// activation rows fill the LDS at a third of K or less, so they split K; the split partials are
// plain stores, summed in split order by a second, fully parallel kernel that also runs the
// epilogue (a last arriver would serialise several items' sums per wave).
#include "bvf_impl.hpp"

#include <algorithm>
#include <cmath>
#include <mutex>
#include <unordered_map>

namespace bvf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kSlotQ4 = 1280;     // codes 1024 B + scale|min 256 B per (tile, superblock)
constexpr int kSlotBf16 = 4096;   // 16 columns x 128 bf16

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
    int S, sb_per_split, n_tiles, n_cols;
    int ring_slots;   // LDS slots per wave ring (R)
    int KS;           // K parts per tile inside a workgroup (waves per tile)
    int T;            // tiles per workgroup item (waves / KS)
    // host-computed reciprocals, so the kernel divides without an integer-division sequence:
    // n / KS = (n * mag_ks) >> 16 for n < 4096, n / stride = (n * mag_stride) >> 32 for n < 65536
    uint32_t mag_ks;
    uint64_t mag_stride;
    int half;   // STORE on a gate|up image: -1 all 16 columns, 0 the gate half, 1 the up half
    // RMSNorm folded into the staging of A (xsrc != nullptr): A = bf16(x * rinv * gain) with
    // rinv = 1 / sqrt(sum(ss_in[m][0 .. n_ss)) / K + eps), for rows m < NF (NF = M unless a mixed
    // staging folds only the first rows); rows NF .. M - 1 are copied from A
    const float* xsrc;
    int NF;
    int ldx;
    const float* ss_in;
    int n_ss;
    const uint16_t* gain;
    float eps;
    float* ss_out;   // STORE / RESID: per row and 16-column tile, the sum of squares of the outputs
    const uint16_t* rscale;   // RESID: the updated rows are scaled by this bf16 value (nullptr: not)
    const int32_t* tokens;    // PLE: row m multiplies by the bf16 ple[clamp(tokens[m]) * ple_ld + n]
    const uint16_t* ple;
    int ple_ld, vocab;
};

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32; NaN stays a NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float half_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// (x & m) | o in one VALU op (m in a scalar register, o in a vector register).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
    return r;
}

// Sum over the four lanes of a quad (lanes 4i .. 4i + 3) with DPP quad permutations.
__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));   // lane ^ 1
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));   // lane ^ 2
    return v;
}

// Sum over all 64 lanes without LDS traffic: the 16-lane rows by DPP (quad swaps, half-row and
// row mirrors), then the four row sums in row order; every lane gets the same bits.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    const int b = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) + __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) + __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

__device__ __forceinline__ float bf16x8_sum(const u32x4& o) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) s += __builtin_bit_cast(float, o[q] << 16) + __builtin_bit_cast(float, o[q] & 0xffff0000u);
    return s;
}

// s_waitcnt with only the vector-memory count (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_lds() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier over LDS traffic only: this wave's LDS reads and writes are complete, then
// s_barrier. (__syncthreads also waits for every outstanding global load, the weight ring's
// included, which would serialise the ring fill with the staging.)
__device__ __forceinline__ void lds_barrier() {
    wait_lds();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Eight 16-byte LDS reads that the compiler's wait-count insertion does not see, issued together and
// complete when the asm block ends (so no output register is in flight past it; the outputs are
// early-clobber, since an address is read after earlier reads are issued). A plain LDS read of a
// region that direct global->LDS copies wrote makes the compiler wait for every outstanding global
// load first, the weight ring's included; the caller orders these reads itself (the copies they
// depend on are complete after its own wait and a barrier).
__device__ __forceinline__ void lds_read16x8_untracked(u32x4 (&o)[8], const void* const (&p)[8]) {
    uint32_t ad[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) ad[r] = (uint32_t)(uintptr_t)(lds_void*)p[r];
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
        : "memory");
}

// Direct loads of one (tile, superblock) of weights into a ring slot of this wave. The slot's
// index idx = tile * TG + superblock (TG = G for Q4_1, 16 G for bf16 rows) is wave-uniform: the
// address arithmetic stays scalar and each lane adds its fixed offset.
template <int FMT>
__device__ __forceinline__ void issue_slot(const KArgs& a, int idx, uint8_t* slot, int lane) {
    const size_t u = (size_t)__builtin_amdgcn_readfirstlane(idx);
    if constexpr (FMT == W_Q4_1) {
        __builtin_amdgcn_global_load_lds((const void*)((const u32x4*)a.codes + u * 64 + lane), (lds_void*)slot, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)((const uint32_t*)a.sm + u * 64 + lane), (lds_void*)(slot + 1024), 4, 0, 0);
    } else {
        const int c = lane & 15, sub = lane >> 4;
        const uint16_t* row = (const uint16_t*)a.codes + u * kSuper + (size_t)c * a.K + sub * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(row + j * 32), (lds_void*)(slot + j * 1024), 16, 0, 0);
    }
}
template <int FMT>
constexpr int loads_per_slot() { return FMT == W_Q4_1 ? 2 : 4; }

// One superblock from a ring slot for MT row tiles. A (this lane's row of tile t, 4 blocks of 8
// bf16) comes from the LDS copy of the rows at As_k + a_off[t]; lanes of rows >= M read row 0.
//
// Q4_1: block j contributes scale_j * C'_j (bf16 MFMA + VALU FMAs) and the min terms of the four
// blocks are one fp32 MFMA 16x16x4 into accm, fed by the block sums the staging step left in LDS
// (this lane's value for tile t: S[m = 16 t + lane % 16][j = lane / 16]) and MM[j][c] = min - 16 scale.
// The dequantised B operand of a block is built once and used by the MT tiles.
template <int FMT, int MT>
__device__ __forceinline__ void compute_slot(const uint8_t* slot, const uint16_t* As_k, const int (&a_off)[MT],
                                             const float (&s_val)[MT], int lane, floatx4 (&acc)[MT],
                                             floatx4 (&accm)[MT]) {
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    const int c = lane & 15, sub = lane >> 4;
    u32x4 av4[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) av4[t][j] = *(const u32x4*)(As_k + a_off[t] + j * 32);
    if constexpr (FMT == W_Q4_1) {
        const u32x4 cw = *(const u32x4*)(slot + lane * 16);
        const u32x4 sm = *(const u32x4*)(slot + 1024 + c * 16);
        const uint32_t smj = *(const uint32_t*)(slot + 1024 + (c * 4 + sub) * 4);   // column c, block sub
        const float mm = fmaf(-16.f, half_lo(smj), half_hi(smj));
#pragma unroll
        for (int t = 0; t < MT; ++t) accm[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(s_val[t], mm, accm[t], 0, 0, 0);
        // block j's MFMAs are issued before block j-1's scale FMAs (covers the MFMA latency with two
        // blocks of results live; the sched barriers keep the scheduler from hoisting all MFMAs)
        floatx4 cc[MT][2];
        uint32_t O;   // bf16 pair 16 | 16 with the code bits clear; the nibble lands in mantissa bits 3..6
        asm("v_mov_b32 %0, 0x41804180" : "=v"(O));
        const uint32_t M4 = 0x00780078u;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            if (j < 4) {
                const uint32_t w = cw[j];
                const u32x4 b = {and_or(w << 3, M4, O), and_or(w >> 1, M4, O), and_or(w >> 5, M4, O), and_or(w >> 9, M4, O)};
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    cc[t][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av4[t][j]),
                                                                           __builtin_bit_cast(bf16x8, b), zero, 0, 0, 0);
            }
            if (j > 0) {
                const int jp = j - 1;
                const float s = half_lo(sm[jp]);
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(s, cc[t][jp & 1][r], acc[t][r]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        (void)s_val; (void)accm; (void)c; (void)sub;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 bw = *(const u32x4*)(slot + j * 1024 + lane * 16);
#pragma unroll
            for (int t = 0; t < MT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av4[t][j]), __builtin_bit_cast(bf16x8, bw),
                                                                 acc[t], 0, 0, 0);
        }
    }
}

// RESID rows of a tile, loaded ahead (the split-K tail issues them before its arrival)
__device__ __forceinline__ floatx4 load_resid_rows(const KArgs& a, int tile, int lane, int m0) {
    const int c = lane & 15, sub = lane >> 4;
    floatx4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = m0 + 4 * sub + r;
        y[r] = m < a.M ? a.y[(size_t)m * a.ldy + tile * kTile + c] : 0.f;
    }
    return y;
}

// Output rows m0 + 4 sub + r of the tile (m0: the row tile's first row).
template <int EPI>
__device__ __forceinline__ void epilogue(const KArgs& a, const floatx4& acc, int tile, int lane, int m0,
                                         bool have_pre = false, floatx4 y_pre = {0.f, 0.f, 0.f, 0.f}) {
    const int c = lane & 15, sub = lane >> 4;
    const int n = tile * kTile + c;
    if constexpr (EPI == EPI_PLE) {
        // the per-layer embedding gate: silu of the GEMM output times the row's per-layer input
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 4 * sub + r;
            if (m >= a.M) continue;
            int t = a.tokens[m];
            t = t < 0 ? 0 : (t >= a.vocab ? a.vocab - 1 : t);
            const float p = __builtin_bit_cast(float, (uint32_t)a.ple[(size_t)t * a.ple_ld + n] << 16);
            const float g = acc[r];
            a.out[(size_t)m * a.ldo + n] = f32_to_bf16(g / (1.0f + expf(-g)) * p);
        }
        return;
    }
    if constexpr (EPI == EPI_SWIGLU) {
        // a gate|up tile holds gate columns in lanes c < 8 and the matching up columns in c + 8
        floatx4 up;
#pragma unroll
        for (int r = 0; r < 4; ++r) up[r] = __shfl_xor(acc[r], 8);
        if (c < 8) {
            const int nh = tile * 8 + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 4 * sub + r;
                if (m >= a.M) continue;
                const float g = acc[r];
                a.out[(size_t)m * a.ldo + nh] = f32_to_bf16(g / (1.0f + expf(-g)) * up[r]);
            }
        }
        return;
    }
    float vout[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = m0 + 4 * sub + r;
        vout[r] = 0.f;
        if (m >= a.M) continue;
        if constexpr (EPI == EPI_STORE) {
            vout[r] = acc[r];
            if (a.half < 0) {
                a.y[(size_t)m * a.ldy + n] = acc[r];
            } else if ((c >> 3) == a.half) {
                a.y[(size_t)m * a.ldy + tile * 8 + (c & 7)] = acc[r];
            }
        } else {
            float v = (have_pre ? y_pre[r] : a.y[(size_t)m * a.ldy + n]) + acc[r];
            if (a.rscale) v *= __builtin_bit_cast(float, (uint32_t)a.rscale[0] << 16);
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
            const int m = m0 + 4 * sub + r;
            if (c == 0 && m < a.M) a.ss_out[(size_t)m * (a.n_cols / kTile) + tile] = q;
        }
    }
}

// Split-K: every wave stores its partial tile at device scope (sc1) as soon as the tile's K range
// is done. After its whole stream the wave waits until its stores are performed, bumps the arrival
// counter of each of its tiles, and for the tiles where it arrived last reads the S partials at
// device scope and sums them in split order (the hardware guarantee this relies on is stated at
// the hand-off).
__device__ __forceinline__ void splitk_store(const KArgs& a, const floatx4& acc, int tile, int split, int lane, int m0) {
    const int c = lane & 15, sub = lane >> 4;
    const int n = tile * kTile + c;
    float* P = a.partial + (size_t)split * a.M * a.n_cols;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = m0 + 4 * sub + r;
        if (m < a.M) __hip_atomic_store(P + (size_t)m * a.n_cols + n, acc[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__device__ __forceinline__ floatx4 splitk_sum(const KArgs& a, int tile, int lane, int m0) {
    const int c = lane & 15, sub = lane >> 4;
    const float* base = a.partial + tile * kTile + c;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    // the loads of four splits of the four rows go out together (one round for S <= 4); the sums
    // run in split order
    for (int sp0 = 0; sp0 < a.S; sp0 += 4) {
        float v[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 4 * sub + r < a.M ? m0 + 4 * sub + r : 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[r][i] = sp0 + i < a.S
                              ? __hip_atomic_load(base + ((sp0 + i) * a.M + m) * a.n_cols, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                              : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[r] += v[r][i];
    }
    return acc;
}

// Wide chunks: plain stores of a split's partial tile (k_splitk_epilogue reads them after the
// kernel boundary).
__device__ __forceinline__ void splitk_store_plain(const KArgs& a, const floatx4& acc, int tile, int split, int lane, int m0) {
    const int c = lane & 15, sub = lane >> 4;
    const int n = tile * kTile + c;
    float* P = a.partial + (size_t)split * a.M * a.n_cols;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = m0 + 4 * sub + r;
        if (m < a.M) P[(size_t)m * a.n_cols + n] = acc[r];
    }
}

// Wide chunks, second kernel: the S partials of every output summed in split order, then the
// GEMM's epilogue. One wave per (4 rows, 64 columns): lane l owns column 64 g + l of the 4 rows,
// so each load of a partial row reads 256 contiguous bytes (the MFMA layout would read 64-byte
// pieces); the epilogue's 16-column tiles are groups of 16 lanes (n_cols is a multiple of 16), whose
// gate/up halves and per-tile sums of squares meet by shuffles inside the group.
template <int EPI>
__global__ __launch_bounds__(256) void k_splitk_epilogue(KArgs a, int n_rt) {
    const int lane = threadIdx.x & 63;
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int n_cg = (a.n_cols + 63) >> 6;
    if (wv >= n_cg * n_rt) return;   // uniform in the wave
    const int cg = wv / n_rt, rt = wv - cg * n_rt;
    const int n = cg * 64 + lane;
    const bool live = n < a.n_cols;            // whole 16-lane groups
    const int c = lane & 15, tile = n >> 4;
    constexpr int RE = 4;
    const int m0 = RE * rt, nr = min(RE, a.M - m0);   // rows of this wave (uniform)
    const float* col = a.partial + (live ? n : 0);
    float acc[RE];
#pragma unroll
    for (int r = 0; r < RE; ++r) acc[r] = 0.f;
    // the loads of four splits go out together; the sums run in split order
    for (int sp0 = 0; sp0 < a.S; sp0 += 4) {
        float v[4][RE];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float* ps = col + (size_t)min(sp0 + i, a.S - 1) * a.M * a.n_cols;
#pragma unroll
            for (int r = 0; r < RE; ++r) v[i][r] = ps[(size_t)(m0 + (r < nr ? r : nr - 1)) * a.n_cols];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < RE; ++r) acc[r] += sp0 + i < a.S ? v[i][r] : 0.f;
    }
    float yp[RE];   // RESID: the residual rows, loaded together
    if constexpr (EPI == EPI_RESID) {
#pragma unroll
        for (int r = 0; r < RE; ++r) yp[r] = a.y[(size_t)(m0 + (r < nr ? r : nr - 1)) * a.ldy + (live ? n : 0)];
    }
    const float rs = EPI == EPI_RESID && a.rscale ? __builtin_bit_cast(float, (uint32_t)a.rscale[0] << 16) : 1.f;
#pragma unroll
    for (int r = 0; r < RE; ++r) {
        if (r >= nr) break;
        const int m = m0 + r;
        const float v = acc[r];
        if constexpr (EPI == EPI_PLE) {
            if (live) {
                int t = a.tokens[m];
                t = t < 0 ? 0 : (t >= a.vocab ? a.vocab - 1 : t);
                const float p = __builtin_bit_cast(float, (uint32_t)a.ple[(size_t)t * a.ple_ld + n] << 16);
                a.out[(size_t)m * a.ldo + n] = f32_to_bf16(v / (1.0f + expf(-v)) * p);
            }
            continue;
        }
        if constexpr (EPI == EPI_SWIGLU) {
            // gate columns in lanes c < 8 of a tile, the matching up columns in c + 8
            const float up = __shfl_xor(v, 8);
            if (live && c < 8) a.out[(size_t)m * a.ldo + tile * 8 + c] = f32_to_bf16(v / (1.0f + expf(-v)) * up);
            continue;
        }
        float vo;
        if constexpr (EPI == EPI_STORE) {
            vo = v;
            if (live) {
                if (a.half < 0) a.y[(size_t)m * a.ldy + n] = v;
                else if ((c >> 3) == a.half) a.y[(size_t)m * a.ldy + tile * 8 + (c & 7)] = v;
            }
        } else {
            float w = yp[r] + v;
            if (a.rscale) w *= rs;
            vo = w;
            if (live) {
                a.y[(size_t)m * a.ldy + n] = w;
                if (a.taps) a.taps[(size_t)m * a.ldt + n] = f32_to_bf16(w);
            }
        }
        if (a.ss_out) {
            float q = vo * vo;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) q += __shfl_xor(q, o);
            if (live && c == 0) a.ss_out[(size_t)m * (a.n_cols / kTile) + tile] = q;
        }
    }
}

// Workgroup (u, split) of the grid U x S and W = blockDim / 64 waves: split = the cross-workgroup
// K split, u = its index among the U workgroups of that split. The W waves are T = W / KS tiles times KS parts
// of the split's K range (wave w: tile slot w / KS, part w % KS). Item i of the workgroup covers
// tiles (u + i U) T + 0 .. T - 1; the KS partial tiles of an item are summed in LDS in part order.
// Rows >= M of the MFMA tiles read arbitrary LDS data: they only feed output rows that are never
// stored. MT row tiles of 16 (M <= 16 MT); MT > 1 workgroups hold at most 8 waves.
template <int FMT, int EPI, int R, int MT>
__global__ __launch_bounds__(MT == 1 ? 1024 : 512) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 4 : 2, 8))) void k_gemm(KArgs a) {
    // dynamic LDS: [ring: W waves x ring_slots slots] [Q4_1: block sums S[sb_per_split * 4][16 MT] fp32]
    //              [A: M rows x lds_ld bf16] [KS > 1: partial tiles W x 64 lanes x MT x 4 fp32]
    constexpr int MP = 16 * MT;   // rows of the block-sum table
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
    constexpr int SLOT = FMT == W_Q4_1 ? kSlotQ4 : kSlotBf16;
    constexpr int LPS = loads_per_slot<FMT>();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: loop control stays scalar
    const int nw = blockDim.x >> 6;
    const int nthr = blockDim.x;
    const int KS = a.KS, T = a.T;
    const int ts = (int)(((uint32_t)wave * a.mag_ks) >> 16), kp = wave - ts * KS;
    const int S = a.S;
    const int split = blockIdx.y;
    const int u = blockIdx.x;
    const int U = gridDim.x;
    const int g0 = split * a.sb_per_split;
    const int nsb = min(a.G, g0 + a.sb_per_split) - g0;
    const int spk = (int)(((uint32_t)(nsb + KS - 1) * a.mag_ks) >> 16);
    const int kb0 = min(nsb, kp * spk), nkp = min(nsb, kb0 + spk) - kb0;   // this wave's superblocks
    const int lds_ld = a.sb_per_split * kSuper + 8;
    uint8_t* ring = lds_raw + (size_t)wave * a.ring_slots * SLOT;
    float* Ss = (float*)(lds_raw + (size_t)nw * a.ring_slots * SLOT);
    uint16_t* As = (uint16_t*)((uint8_t*)Ss + (FMT == W_Q4_1 ? (size_t)a.sb_per_split * 4 * MP * 4 : 0));
    float* red = (float*)(As + (size_t)a.M * lds_ld);

    const int first = u * T;            // first tile of item 0
    const int stride = U * T;           // tiles between items
    auto div_stride = [&](int n) { return (int)(((uint64_t)(uint32_t)n * a.mag_stride) >> 32); };
    const int items = first < a.n_tiles ? div_stride(a.n_tiles - 1 - first) + 1 : 0;   // uniform in the workgroup
    // this wave's valid items: tile = first + i stride + ts < n_tiles
    const int my_items = first + ts < a.n_tiles ? div_stride(a.n_tiles - 1 - first - ts) + 1 : 0;
    const int total = my_items * nkp;   // superblocks this wave streams

    // bf16 activation rows: direct global->LDS copies (1 KB = 4 superblocks of one row per
    // instruction), issued before the ring so the wave's first wait covers them
    const int chunks = (nsb + 3) / 4;
    const int NF = a.xsrc ? a.NF : 0;   // rows [0, NF) normalised from xsrc, [NF, M) copied from A
    if (NF < a.M) {
        int m = NF, q = wave;   // copy i = (m - NF) chunks + q, i = wave, wave + nw, ...
        while (q >= chunks) { q -= chunks; ++m; }
        for (; m < a.M; q += nw) {
            while (q >= chunks) { q -= chunks; ++m; }
            if (m >= a.M) break;
            const int e = q * 512 + lane * 8;   // element offset in the K range
            if (e < nsb * kSuper)
                __builtin_amdgcn_global_load_lds((const void*)(a.A + (size_t)m * a.lda + (size_t)g0 * kSuper + e),
                                                 (lds_void*)(As + m * lds_ld + q * 512), 16, 0, 0);
        }
    }
    // RMSNorm folded in. Work items (piece p = 8 elements of the K range, batch b of RG rows), item
    // i = b pieces + p, thread t takes items t, t + nthr, ...; the loads of the first item (the RG
    // rows' pieces and the gains) and of the rows' sums of squares go out before the ring, so they are
    // not queued behind the weight stream. When the items leave waves without a first item, those
    // waves come first and compute the rows' factors rinv (their few loads go out ahead of the rows'),
    // and the converting waves pass the barrier that publishes rinv without waiting for their own
    // loads. Otherwise every wave computes its rows' factors once all its loads are in.
    __shared__ float rinv_s[kMaxGemmRows];
    constexpr int RG = 4;
    const int pieces = nsb * (kSuper / 8);
    const int n_items = a.xsrc ? pieces * ((NF + RG - 1) / RG) : 0;
    const int conv_waves = min(nw, (n_items + 63) >> 6);   // waves that hold a first item
    const int n_rw = nw - conv_waves;                      // > 0: waves 0 .. n_rw - 1 compute rinv
    const int p0 = (int)threadIdx.x - 64 * n_rw;            // the thread's first item (< 0: none)
    const bool has0 = p0 >= 0 && p0 < n_items;
    const int b0 = has0 ? p0 / pieces : 0, pp0 = has0 ? p0 - b0 * pieces : 0;
    const int rw_n = n_rw > 0 ? n_rw : nw;
    const int rw_idx = wave;
    const bool my_rinv = n_rw == 0 || wave < n_rw;         // uniform in the wave
    float4 xv[RG][2];
    u32x4 gv0 = {0u, 0u, 0u, 0u};
    float sv[4][4];   // sums of squares of rows rw_idx + rw_n r (r < 4), lanes lane + 64 t (t < 4)
    if (a.xsrc) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = rw_idx + rw_n * r;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int i = lane + 64 * t;
                sv[r][t] = my_rinv && m < NF && i < a.n_ss ? a.ss_in[(size_t)m * a.n_ss + i] : 0.f;
            }
        }
        if (has0) {
            const int k0 = g0 * kSuper + pp0 * 8;
            gv0 = *(const u32x4*)(a.gain + k0);
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const int m = min(RG * b0 + r, NF - 1);
                xv[r][0] = *(const float4*)(a.xsrc + (size_t)m * a.ldx + k0);
                xv[r][1] = *(const float4*)(a.xsrc + (size_t)m * a.ldx + k0 + 4);
            }
        }
    }
    // RESID without a K split: the residual rows of the wave's first item are loaded before the ring,
    // so the epilogue does not wait for them (they land with the staging loads)
    floatx4 y_first = {0.f, 0.f, 0.f, 0.f};
    const bool y_early = EPI == EPI_RESID && MT == 1 && S == 1 && kp == 0 && my_items > 0;
    if (y_early) y_first = load_resid_rows(a, first + ts, lane, 0);
    // fill the ring: the weight loads overlap the staging of the activation rows. Exactly R slots
    // are filled (slots past the wave's stream repeat its first superblock, an L2 hit, and are never
    // read), so the staging's own waits can count the copies that follow its loads.
    asm volatile("" ::: "memory");   // the staging loads above leave before the weight copies
    __builtin_amdgcn_sched_barrier(0);
    // slot index of the next copy (uniform): +1 per superblock, + wrap from an item's last
    // superblock to the next item's first; a wave with nothing to stream repeats a valid index
    const int TG = FMT == W_Q4_1 ? a.G : kTile * a.G;
    int ib = total > 0 ? (a.tile0 + (first + ts) * a.tile_stride) * TG + g0 + kb0 : a.tile0 * TG + g0;
    const int ib_first = ib;
    const int ib_wrap = stride * a.tile_stride * TG - (nkp - 1);
    int is_g = 0;
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const bool real = t < total;
        issue_slot<FMT>(a, real ? ib : ib_first, ring + t * SLOT, lane);
        if (real) {
            if (++is_g == nkp) { is_g = 0; ib += ib_wrap; }
            else ++ib;
        }
    }
    int s_issue = total < R ? total : R;

    // block sums S[b][m] = sum of the 32 bf16 of block b of row m for the copied rows NF .. M - 1 (the
    // normalised rows get theirs while being converted); the four pieces of a block sit in four
    // consecutive lanes; eight rows' LDS reads are issued together; work items (piece p, 8-row batch b
    // from row NF). Called on each staging path separately, so that neither path's pending loads
    // reach the other's code.
    auto copied_block_sums = [&]() __attribute__((always_inline)) {
        const int n_cb = pieces * ((a.M - NF + 7) >> 3);
        for (int i = threadIdx.x; i < n_cb; i += nthr) {
            const int b = i / pieces, p = i - b * pieces;
            const int m0 = NF + 8 * b;
            u32x4 o[8];
            const void* src[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) src[r] = As + (m0 + r < a.M ? m0 + r : m0) * lds_ld + p * 8;
            lds_read16x8_untracked(o, src);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float bs = quad_sum(bf16x8_sum(o[r]));
                if (m0 + r < a.M && (p & 3) == 0) Ss[(p >> 2) * MP + m0 + r] = bs;
            }
        }
    };
    if (a.xsrc) {
        if (my_rinv) {
            // the sums of squares have returned once only the R ring slots are younger (without
            // rinv waves, this wave's first item's loads too)
            wait_vm<LPS * R>();
            // rinv from the producer's per-tile sums of squares (n_ss > 256 continues in a loop)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = rw_idx + rw_n * r;
                if (m >= NF) break;
                float q = (sv[r][0] + sv[r][1]) + (sv[r][2] + sv[r][3]);
                for (int i = lane + 256; i < a.n_ss; i += 64) q += a.ss_in[(size_t)m * a.n_ss + i];
                q = wave_sum_dpp(q);
                if (lane == 0) rinv_s[m] = 1.0f / sqrtf(q / (float)a.K + a.eps);
            }
            // rows past 4 rw_n (wide chunks): the same sums, loaded now
            for (int m = rw_idx + 4 * rw_n; m < NF; m += rw_n) {
                float t4[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int i = lane + 64 * t;
                    t4[t] = i < a.n_ss ? a.ss_in[(size_t)m * a.n_ss + i] : 0.f;
                }
                float q = (t4[0] + t4[1]) + (t4[2] + t4[3]);
                for (int i = lane + 256; i < a.n_ss; i += 64) q += a.ss_in[(size_t)m * a.n_ss + i];
                q = wave_sum_dpp(q);
                if (lane == 0) rinv_s[m] = 1.0f / sqrtf(q / (float)a.K + a.eps);
            }
        }
        lds_barrier();
        auto convert = [&](int p, int m0, int nrows, const u32x4& gv, const float4 (&xr)[RG][2]) {
            float rvs[RG];   // the rows' factors in registers before any LDS write of the batch
#pragma unroll
            for (int r = 0; r < RG; ++r) rvs[r] = rinv_s[m0 + r];
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                if (r >= nrows) break;
                const int m = m0 + r;
                const float rv = rvs[r];
                const float xs[8] = {xr[r][0].x, xr[r][0].y, xr[r][0].z, xr[r][0].w, xr[r][1].x, xr[r][1].y, xr[r][1].z, xr[r][1].w};
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float g_lo = __builtin_bit_cast(float, gv[q] << 16);
                    const float g_hi = __builtin_bit_cast(float, gv[q] & 0xffff0000u);
                    o[q] = pack_bf16x2(xs[2 * q] * rv * g_lo, xs[2 * q + 1] * rv * g_hi);
                }
                *(u32x4*)(As + m * lds_ld + p * 8) = o;
                if constexpr (FMT == W_Q4_1) {
                    // block sum of the 32 bf16 of block p / 4 (the quad of lanes holding its pieces)
                    const float bs = quad_sum(bf16x8_sum(o));
                    if ((p & 3) == 0) Ss[(p >> 2) * MP + m] = bs;
                }
            }
        };
        // the first item, loaded above (its loads are in once only the ring slots are younger); the
        // four pieces of a block sit in four consecutive lanes (pieces and the thread count are
        // multiples of 4)
        if (has0) {
            wait_vm<LPS * R>();
            convert(pp0, RG * b0, min(RG, NF - RG * b0), gv0, xv);
        }
        for (int i = p0 + nthr; i < n_items; i += nthr) {   // (none when there are rinv waves)
            const int b = i / pieces, p = i - b * pieces;
            const int m0 = RG * b, nrows = min(RG, NF - m0);
            const int k0 = g0 * kSuper + p * 8;
            const u32x4 gv = *(const u32x4*)(a.gain + k0);
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const int m = m0 + (r < nrows ? r : nrows - 1);
                xv[r][0] = *(const float4*)(a.xsrc + (size_t)m * a.ldx + k0);
                xv[r][1] = *(const float4*)(a.xsrc + (size_t)m * a.ldx + k0 + 4);
            }
            convert(p, m0, nrows, gv, xv);
        }
        // every staging load of the wave has returned by now; the wait says so to the compiler
        wait_vm<LPS * R>();
        lds_barrier();
        if (FMT == W_Q4_1 && NF < a.M) {
            copied_block_sums();
            lds_barrier();
        }
    } else {
        // this wave's activation copies have landed (they are older than its R ring slots)
        wait_vm<LPS * R>();
        lds_barrier();
        if (FMT == W_Q4_1) {
            copied_block_sums();
            lds_barrier();
        }
    }
    if (items == 0) return;   // uniform in the workgroup

    const int m_a = lane & 15, sub = lane >> 4;
    int a_off[MT];   // this lane's A row in row tile t (rows >= M read row 0)
#pragma unroll
    for (int t = 0; t < MT; ++t) a_off[t] = (16 * t + m_a < a.M ? 16 * t + m_a : 0) * lds_ld;
    const uint16_t* As_k = As + sub * 8 + kb0 * kSuper;
    // block sum of superblock i of this wave's part for row tile t: Ss_l[4 MP i + 16 t]
    const float* Ss_l = Ss + m_a + sub * MP + 4 * MP * kb0;

    int s_off = 0;   // ring offset of the next slot to use
    uint32_t last = 0;   // split-K: bit i set where this wave arrived last on item i (reducer waves)
    for (int it = 0; it < items; ++it) {
        const int tile = first + it * stride + ts;
        floatx4 acc[MT], accm[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = accm[t] = (floatx4){0.f, 0.f, 0.f, 0.f};
        if (it < my_items) {
#pragma nounroll
            for (int gi = 0; gi < nkp; ++gi) {
                // R slots are always in flight (past the stream's end the refills repeat a valid
                // superblock into the slot just used), so the oldest has landed at R - 1 younger
                wait_vm<LPS * (R - 1)>();
                uint8_t* slot = ring + s_off;
                float s_val[MT];
#pragma unroll
                for (int t = 0; t < MT; ++t) s_val[t] = FMT == W_Q4_1 ? Ss_l[4 * MP * gi + 16 * t] : 0.f;
                compute_slot<FMT, MT>(slot, As_k + gi * kSuper, a_off, s_val, lane, acc, accm);
                wait_lds();   // the slot's LDS reads have returned before the refill overwrites it
                const bool real = s_issue < total;
                issue_slot<FMT>(a, real ? ib : ib_first, slot, lane);
                if (real) {
                    ++s_issue;
                    if (++is_g == nkp) { is_g = 0; ib += ib_wrap; }
                    else ++ib;
                }
                s_off = s_off + SLOT == R * SLOT ? 0 : s_off + SLOT;
            }
            if constexpr (FMT == W_Q4_1) {
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[t] += accm[t];
            }
        }
        if (KS > 1) {
            // the KS parts of each tile meet in LDS; part 0 sums them in part order
#pragma unroll
            for (int t = 0; t < MT; ++t) *(floatx4*)(red + (((size_t)wave * 64 + lane) * MT + t) * 4) = acc[t];
            lds_barrier();
            if (kp == 0) {
                for (int q = 1; q < KS; ++q)
#pragma unroll
                    for (int t = 0; t < MT; ++t) acc[t] += *(const floatx4*)(red + (((size_t)(wave + q) * 64 + lane) * MT + t) * 4);
            }
            lds_barrier();
        }
        if (kp != 0 || it >= my_items) continue;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (16 * t >= a.M) break;
            if (S == 1) epilogue<EPI>(a, acc[t], tile, lane, 16 * t, y_early && it == 0, y_first);
            else if (MT > 1) splitk_store_plain(a, acc[t], tile, split, lane, 16 * t);
            else splitk_store(a, acc[t], tile, split, lane, 16 * t);
        }
    }
    wait_vm<0>();   // no copy into this wave's ring is left in flight
    if (MT == 1 && S > 1 && kp == 0 && my_items > 0) {
        // a single item's residual rows are loaded now, in the shadow of the stores and the arrival
        floatx4 y_pre = {0.f, 0.f, 0.f, 0.f};
        if (EPI == EPI_RESID && MT == 1 && my_items == 1) y_pre = load_resid_rows(a, first + ts, lane, 0);
        // The hand-off relies on what gfx950 does with device-scope (sc1) relaxed atomics, not on
        // release/acquire fences: agent-scope release/acquire fences write back and invalidate the
        // whole L2 of the XCD (buffer_wbl2 / buffer_inv), which made each down launch 5 us slower.
        //  - the partial stores and loads are device-scope atomics, coherent across the XCDs (the
        //    compiler emits them with the sc1 scope bit; each location has one modification order
        //    at device scope), so no L2 writeback or invalidation is needed for them;
        //  - s_waitcnt 0 waits until every store of the wave is acknowledged as performed, before
        //    the arrival atomic is issued (the compiler barriers keep the compiler from moving
        //    memory operations across it);
        //  - the last arriver issues its partial loads (device-scope atomic loads, read at the
        //    coherence point) only after its arrival returned S - 1, i.e. after every other split's
        //    arrival, each of which followed that split's performed stores.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        if (lane == 0) {
            for (int it = 0; it < my_items; ++it)
                if (__hip_atomic_fetch_add(&a.counters[first + it * stride + ts], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1)
                    last |= 1u << it;
        }
        last = __shfl(last, 0);
        asm volatile("" ::: "memory");
        for (int it = 0; it < my_items; ++it) {
            if (!((last >> it) & 1u)) continue;
            const int tile = first + it * stride + ts;
            for (int t = 0; t < MT && 16 * t < a.M; ++t)
                epilogue<EPI>(a, splitk_sum(a, tile, lane, 16 * t), tile, lane, 16 * t,
                              EPI == EPI_RESID && MT == 1 && my_items == 1, y_pre);
            if (lane == 0) __hip_atomic_store(&a.counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int FMT, int EPI, int R, int MT>
hipError_t launch_r(const KArgs& k, int grid, int waves, size_t lds, hipStream_t st) {
    const dim3 g2((unsigned)(grid / k.S), (unsigned)k.S);   // U workgroups per split, S splits
    if (waves * 64 > (MT == 1 ? 1024 : 512)) return hipErrorInvalidValue;
    static bool attr_set = false;   // raise the dynamic LDS limit once per instantiation
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)k_gemm<FMT, EPI, R, MT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)kGemmLdsMax);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((k_gemm<FMT, EPI, R, MT>), g2, dim3(64 * waves), lds, st, k);
    if constexpr (MT > 1) {
        if (k.S > 1) {
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int n_rt = (k.M + 3) / 4;   // groups of 4 rows (the summing kernel's waves)
            const int waves_total = (k.n_cols + 63) / 64 * n_rt;
            hipLaunchKernelGGL(k_splitk_epilogue<EPI>, dim3((waves_total + 3) / 4), dim3(256), 0, st, k, n_rt);
        }
    }
    return hipGetLastError();
}

// MT > 1 (wide chunks): Q4_1 only, rings of 2 superblocks (measured on MI355X at 64 rows: rings of
// 4 leave room for fewer waves and the prefill ran 10% slower)
template <int FMT, int EPI>
hipError_t launch_fe(int R, int MT, const KArgs& k, int grid, int waves, size_t lds, hipStream_t st) {
    if (MT == 1) {
        switch (R) {
            case 2: return launch_r<FMT, EPI, 2, 1>(k, grid, waves, lds, st);
            case 4: return launch_r<FMT, EPI, 4, 1>(k, grid, waves, lds, st);
            case 8: return launch_r<FMT, EPI, 8, 1>(k, grid, waves, lds, st);
        }
        return hipErrorInvalidValue;
    }
    if constexpr (FMT == W_Q4_1) {
        if (R == 2 && MT == 2) return launch_r<FMT, EPI, 2, 2>(k, grid, waves, lds, st);
        if (R == 2 && MT == 4) return launch_r<FMT, EPI, 2, 4>(k, grid, waves, lds, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t gemm_lds_bytes(int fmt, int M, int sb, int waves, int ring, int KS) {
    const size_t slot = fmt == W_Q4_1 ? kSlotQ4 : kSlotBf16;
    const int mt = gemm_row_tiles(M);
    return (size_t)waves * ring * slot + (fmt == W_Q4_1 ? (size_t)sb * 4 * 16 * mt * 4 : 0) +
           (size_t)M * ((size_t)sb * kSuper + 8) * 2 + (KS > 1 ? (size_t)waves * 1024 * mt : 0);
}

// Plan: choose the cross-workgroup K split S, the waves per workgroup W = T tiles x KS parts, the
// ring depth R, the items per workgroup and the grid. Every workgroup of the grid must be resident
// at once (one round: no tail). Cost estimate per launch: the activation staging (rounds of L2
// loads when the RMSNorm is folded in), the weight stream (bytes at the HBM rate, the wave's
// serial work per superblock, or its superblocks R at a time per memory latency), the in-LDS
// reduction of the parts and the split-K hand-off.
GemmPlan plan_gemm(const GemmLaunch& L) {
    GemmPlan best{};
    best.S = -1;
    const int tiles = L.n_run_tiles, G = L.w.G, M = L.M;
    const int MT = gemm_row_tiles(M);
    const int max_waves = MT == 1 ? 16 : 8;
    const int cus = L.n_cu > 0 ? L.n_cu : 256;
    const size_t slot_bytes = L.fmt == W_Q4_1 ? kSlotQ4 : kSlotBf16;
    const double bytes = (double)tiles * G * slot_bytes;
    // HBM rate, memory latency, compute per superblock and wave, L2 round trip of the staging,
    // split-K hand-off and its cost per split, in-LDS part reduction
    const double hbm = 5.5e12, lat = 1.5e-6, per_sb = 0.25e-6, l2_round = 0.8e-6, handoff = 3.0e-6, per_split = 0.25e-6,
                 reduce = 0.3e-6;
    const bool norm = L.xsrc != nullptr;
    double best_t = 1e30;
    auto consider = [&](int Se, int sb, int W, int KS, int R, int ipw, bool forced) {
        const int T = W / KS;
        const int U = (tiles + T * ipw - 1) / (T * ipw);
        const int spk = (sb + KS - 1) / KS;
        if ((KS - 1) * spk >= sb) return false;   // every K part has superblocks
        const int ring = R;   // every wave fills all R slots once (unused ones with a repeat)
        const size_t lds = gemm_lds_bytes(L.fmt, M, sb, W, ring, KS);
        if (lds > kGemmLdsMax) return false;
        const int wg_cu = (int)std::min<size_t>(16 / W, kLdsPerCu / lds);   // at most 16 waves per CU
        if (wg_cu < 1) return false;
        if (!forced && (long)Se * U > (long)cus * wg_cu) return false;   // not resident in one round
        const double pieces = (double)sb * (kSuper / 8);
        const double staging = norm ? (1.0 + std::ceil(pieces / (64.0 * W)) * std::ceil(M / 8.0)) * l2_round : 0.3e-6;
        const double wsb = (double)ipw * spk;   // superblocks per wave
        // the dequantisation is shared by the MT row tiles; each adds its MFMAs and scale FMAs
        const double sb_cost = per_sb * (1.0 + 0.35 * (MT - 1));
        const double stream = lat + std::max({bytes / hbm, wsb * sb_cost, std::ceil(wsb / R) * lat});
        // the split-K hand-off: arrival, then the last arriver's loads of the Se partials; wide
        // chunks: the partials written and read back by the summing kernel, and its launch
        const double split_t = Se == 1 ? 0.0
                               : MT == 1 ? handoff + Se * per_split
                                         : 2.5e-6 + 2.0 * Se * (double)M * tiles * kTile * 4.0 / 4.0e12;
        const double t = staging + stream + (KS > 1 ? ipw * reduce : 0.0) + split_t;
        if (forced || t < best_t * 0.98) {
            best_t = t;
            best.S = Se;
            best.sb_per_split = sb;
            best.waves = W;
            best.KS = KS;
            best.R = R;
            best.ring_slots = ring;
            best.grid = Se * U;
            best.lds = lds;
        }
        return true;
    };
    int prev_sb = -1;
    for (int S = 1; S <= G && S <= 64; ++S) {
        const int sb = (G + S - 1) / S;
        if (sb == prev_sb) continue;
        prev_sb = sb;
        const int Se = (G + sb - 1) / sb;
        if (Se > 1 && ((size_t)Se * M * tiles * kTile > L.partial_floats || tiles > L.n_counters)) continue;
        for (int W = 4; W <= max_waves; ++W)
            for (int KS = 1; KS <= W; ++KS) {
                if (W % KS) continue;
                for (int R : {8, 4, 2}) {
                    if (L.fmt == W_BF16 && R == 8) continue;
                    // Q4_1 rings hold 2 superblocks: measured on MI355X over every forced plan of the
                    // verify pass's GEMM shapes (q|k|v, o, gate|up, down at k = 8), the best plans
                    // all take rings of 2 and spend the LDS on more waves per workgroup (the
                    // estimate below does not model the ring depth well enough to choose it)
                    if (L.fmt == W_Q4_1 && R != 2) continue;
                    // the fewest items per workgroup for which the grid is resident
                    for (int ipw = 1; ipw <= tiles && (Se == 1 || ipw <= 32); ++ipw)
                        if (consider(Se, sb, W, KS, R, ipw, false)) break;
                }
            }
    }
    // Long K streams staged by copy (the down projections, K >= 64 superblocks): measured on MI355X
    // by the plan sweep at 1, 8 and 16 rows, the best plans split K into parts of about 27
    // superblocks and run 12 waves per workgroup, T tiles x 12 / T parts, with about one workgroup
    // per compute unit; the estimate above does not find them, so they are taken when they fit.
    if (L.fmt == W_Q4_1 && !norm && G >= 64 && L.force_S <= 0 && MT == 1) {
        const int sb = 27, Se = (G + sb - 1) / sb;
        if ((size_t)Se * M * tiles * kTile <= L.partial_floats && tiles <= L.n_counters) {
            for (int T : {1, 2, 3, 4, 6, 12}) {
                const int U = (tiles + T - 1) / T;
                if ((long)Se * U > cus) continue;
                consider(Se, sb, 12, 12 / T, 2, 1, true);
                break;
            }
        }
    }
    // Many tiles over a short K range with the RMSNorm folded in (gate|up of the double-wide
    // layers, >= 8 tiles per compute unit): measured best with one item of T = tiles / n_cu tiles
    // per workgroup and one K part per wave (W = T), one workgroup per compute unit.
    if (L.fmt == W_Q4_1 && norm && L.force_S <= 0 && MT == 1 && tiles % cus == 0 && tiles / cus >= 8 && tiles / cus <= 16)
        consider(1, G, tiles / cus, 1, 2, 1, true);
    // Between one and two tiles per compute unit with the RMSNorm folded in (the draft's q|k|v):
    // measured best with two tiles per workgroup, 8 waves in 4 K parts, at most one workgroup per
    // compute unit (9.4 against 11.1 us for one tile per workgroup of 5 waves).
    if (L.fmt == W_Q4_1 && norm && L.force_S <= 0 && MT == 1 && tiles > cus && tiles <= 2 * cus)
        consider(1, G, 8, 4, 2, 1, true);
    if (L.force_S > 0 && L.force_R > 0 && L.force_ipw > 0 && L.force_W > 0 && L.force_KS > 0 && L.force_W % L.force_KS == 0 &&
        L.force_W <= max_waves) {
        const int sb = (G + L.force_S - 1) / L.force_S;
        const int Se = (G + sb - 1) / sb;
        if (Se == 1 || ((size_t)Se * M * tiles * kTile <= L.partial_floats && tiles <= L.n_counters))
            consider(Se, sb, L.force_W, L.force_KS, L.force_R, L.force_ipw, true);
    }
    return best;
}

// Plans depend only on the launch's shape; the search runs once per shape.
static GemmPlan cached_plan(const GemmLaunch& L) {
    static std::mutex mu;
    static std::unordered_map<uint64_t, GemmPlan> cache;
    uint64_t key = (uint64_t)L.n_run_tiles;
    key = key * 1000003u + (uint64_t)L.w.G;
    key = key * 131u + (uint64_t)L.M;
    key = key * 7u + (uint64_t)(L.fmt * 2 + (L.xsrc != nullptr));
    key = key * 4099u + (uint64_t)L.n_cu;
    key = key * 1000003u + (uint64_t)(L.partial_floats >> 10);
    key = key * 65537u + (uint64_t)L.n_counters;
    key = key * 1000003u + (uint64_t)(((L.force_S * 17 + L.force_R) * 17 + L.force_ipw) * 17 + L.force_W) * 17 + (uint64_t)L.force_KS;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    const GemmPlan p = plan_gemm(L);
    cache.emplace(key, p);
    return p;
}

hipError_t launch_gemm(const GemmLaunch& L, hipStream_t st) {
    if (L.M < 1 || L.M > kMaxGemmRows || (L.M > kMaxRows && L.fmt != W_Q4_1)) return hipErrorInvalidValue;
    const int MT = gemm_row_tiles(L.M);
    const GemmPlan p = cached_plan(L);
    if (p.S < 1) return hipErrorInvalidValue;
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
    k.ring_slots = p.ring_slots;
    k.KS = p.KS;
    k.T = p.waves / p.KS;
    k.mag_ks = (uint32_t)((65536u + p.KS - 1) / p.KS);
    {
        const uint64_t stride = (uint64_t)(p.grid / p.S) * k.T;
        if (L.n_run_tiles >= 65536 || stride >= 65536 || p.waves > 16) return hipErrorInvalidValue;
        k.mag_stride = ((1ull << 32) + stride - 1) / stride;
    }
    k.n_tiles = L.n_run_tiles;
    k.n_cols = L.n_run_tiles * kTile;
    k.half = L.half;
    k.xsrc = L.xsrc;
    k.NF = L.xsrc ? (L.n_fold > 0 && L.n_fold < L.M ? L.n_fold : L.M) : 0;
    k.ldx = L.ldx;
    k.ss_in = L.ss_in;
    k.n_ss = L.n_ss;
    k.gain = L.gain;
    k.eps = L.eps;
    k.ss_out = L.ss_out;
    k.rscale = L.rscale;
    k.tokens = L.tokens;
    k.ple = L.ple;
    k.ple_ld = L.ple_ld;
    k.vocab = L.vocab;
    if (L.epi == EPI_PLE && (!L.tokens || !L.ple || L.vocab < 1 || !L.out)) return hipErrorInvalidValue;
    if (L.fmt == W_Q4_1) {
        switch (L.epi) {
            case EPI_STORE: return launch_fe<W_Q4_1, EPI_STORE>(p.R, MT, k, p.grid, p.waves, p.lds, st);
            case EPI_RESID: return launch_fe<W_Q4_1, EPI_RESID>(p.R, MT, k, p.grid, p.waves, p.lds, st);
            case EPI_SWIGLU: return launch_fe<W_Q4_1, EPI_SWIGLU>(p.R, MT, k, p.grid, p.waves, p.lds, st);
            case EPI_PLE: return launch_fe<W_Q4_1, EPI_PLE>(p.R, MT, k, p.grid, p.waves, p.lds, st);
        }
    } else if (L.epi == EPI_STORE) {
        return launch_fe<W_BF16, EPI_STORE>(p.R, MT, k, p.grid, p.waves, p.lds, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace bvf
