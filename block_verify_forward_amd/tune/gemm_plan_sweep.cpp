// Plan sweep of the small-M Q4_1 GEMM: for each GEMM shape of the target-shaped verify pass (q|k|v of
// a sliding layer, o, gate|up of own and KV-shared layers, down of own and KV-shared layers) and of
// the draft's layers (q|k|v, o, gate|up, down), times
// every forced plan (K splits S, waves W, K parts KS, ring depth R, items per workgroup) that fits
// the LDS, per launch over enough distinct weight copies that the stream comes from HBM (more bytes
// than the 256 MB last-level cache), and checks each plan's output against the planner's own plan.
// Prints the planner's choice and the fastest plans. Synthetic weights (random codes, small finite
// fp16 scale/min) and activations; nothing is read from disk.
//
// build (from the repository root):
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops \
//     -I block_verify_forward_amd/csrc block_verify_forward_amd/tune/gemm_plan_sweep.cpp \
//     block_verify_forward_amd/csrc/gemm.hip -o gemm_plan_sweep
// run: ./gemm_plan_sweep [shape name | all] [rows M, default 8]
#include "bvf_impl.hpp"
#include <cstdio>
#include <cstring>
#include <cstdlib>
#include <vector>
#include <algorithm>
#include <cmath>
#include <string>
using namespace bvf;
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1); } } while (0)
static float bf2f(uint16_t h) { uint32_t u = (uint32_t)h << 16; float f; std::memcpy(&f, &u, 4); return f; }
struct Cls { const char* name; int tiles, G, epi; bool norm; };
int main(int argc, char** argv) {
  const int M = argc > 2 ? atoi(argv[2]) : 8;
  std::vector<Cls> cls = {{"qkv_sliding", 160, 20, EPI_STORE, true}, {"o", 160, 16, EPI_RESID, false},
                          {"gu_own", 1280, 20, EPI_SWIGLU, true}, {"gu_shared", 2560, 20, EPI_SWIGLU, true},
                          {"down_own", 160, 80, EPI_RESID, false}, {"down_shared", 160, 160, EPI_RESID, false},
                          // the draft's layers (hidden 2560, 32 query / 8 KV heads of 128, FFN 5120)
                          {"draft_qkv", 384, 20, EPI_STORE, true}, {"draft_o", 160, 32, EPI_RESID, false},
                          {"draft_gu", 640, 20, EPI_SWIGLU, true}, {"draft_down", 160, 40, EPI_RESID, false}};
  std::string only = argc > 1 && std::string(argv[1]) != "all" ? argv[1] : "";
  const size_t budget = 600ull << 20;   // bytes of weight copies per class
  float* partial; int* counters; CK(hipMalloc(&partial, (16ull << 20) * 4)); CK(hipMalloc(&counters, 16384 * 4));
  CK(hipMemset(counters, 0, 16384 * 4));
  hipStream_t st; CK(hipStreamCreate(&st));
  hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  for (auto& c : cls) {
    if (!only.empty() && only != c.name) continue;
    const int K = c.G * 128, N = c.tiles * 16;
    const size_t cb = (size_t)c.tiles * c.G * 1024, sb = (size_t)c.tiles * c.G * 256;
    const int NC = std::max<int>(2, (int)(budget / (cb + sb)));
    uint8_t *codes, *sm; CK(hipMalloc(&codes, cb * NC)); CK(hipMalloc(&sm, sb * NC));
    {   // codes random, scale|min fp16 pairs: scale 0x2000 + small, min 0xa000 + small (finite)
      std::vector<uint8_t> h(cb); srand(1); for (auto& v : h) v = rand() & 255;
      std::vector<uint32_t> s(sb / 4); for (auto& v : s) v = (0x2000u + (rand() & 0x3ff)) | ((0xa000u + (rand() & 0x3ff)) << 16);
      for (int i = 0; i < NC; ++i) { CK(hipMemcpy(codes + i * cb, h.data(), cb, hipMemcpyHostToDevice)); CK(hipMemcpy(sm + i * sb, s.data(), sb, hipMemcpyHostToDevice)); }
    }
    float *x, *ss, *y, *y0, *ssout; uint16_t *A, *gain, *out;
    CK(hipMalloc(&x, (size_t)M * K * 4)); CK(hipMalloc(&ss, (size_t)M * (K / 16) * 4)); CK(hipMalloc(&A, (size_t)M * K * 2));
    CK(hipMalloc(&gain, (size_t)K * 2)); CK(hipMalloc(&y, (size_t)M * N * 4)); CK(hipMalloc(&y0, (size_t)M * N * 4));
    CK(hipMalloc(&out, (size_t)M * N * 2)); CK(hipMalloc(&ssout, (size_t)M * c.tiles * 4));
    {
      std::vector<float> hx((size_t)M * K); for (auto& v : hx) v = (rand() / (float)RAND_MAX - 0.5f) * 2.f;
      CK(hipMemcpy(x, hx.data(), hx.size() * 4, hipMemcpyHostToDevice));
      std::vector<float> hs((size_t)M * (K / 16), 0.f);
      for (int m = 0; m < M; ++m) for (int t = 0; t < K / 16; ++t) { double q = 0; for (int j = 0; j < 16; ++j) q += (double)hx[(size_t)m * K + t * 16 + j] * hx[(size_t)m * K + t * 16 + j]; hs[(size_t)m * (K / 16) + t] = (float)q; }
      CK(hipMemcpy(ss, hs.data(), hs.size() * 4, hipMemcpyHostToDevice));
      std::vector<uint16_t> ha((size_t)M * K); for (auto& v : ha) v = 0x3f00 | (rand() & 0xff);   // bf16 in [0.5, 1)
      CK(hipMemcpy(A, ha.data(), ha.size() * 2, hipMemcpyHostToDevice));
      std::vector<uint16_t> hg(K, 0x3f80); CK(hipMemcpy(gain, hg.data(), hg.size() * 2, hipMemcpyHostToDevice));
      std::vector<float> hy((size_t)M * N); for (auto& v : hy) v = rand() / (float)RAND_MAX;
      CK(hipMemcpy(y0, hy.data(), hy.size() * 4, hipMemcpyHostToDevice));
    }
    auto mk = [&](int copy) {
      GemmLaunch L; L.w.codes = codes + copy * cb; L.w.sm = sm + copy * sb; L.w.n_tiles = c.tiles; L.w.G = c.G; L.w.K = K;
      L.fmt = W_Q4_1; L.epi = c.epi; L.n_run_tiles = c.tiles; L.M = M; L.partial = partial; L.partial_floats = 16ull << 20;
      L.counters = counters; L.n_counters = 16384; L.n_cu = 256;
      if (c.norm) { L.xsrc = x; L.ldx = K; L.ss_in = ss; L.n_ss = K / 16; L.gain = gain; L.eps = 1e-6f; }
      else { L.A = A; L.lda = K; }
      if (c.epi == EPI_SWIGLU) { L.out = out; L.ldo = N / 2; }
      else { L.y = y; L.ldy = N; L.ss_out = ssout; }
      return L;
    };
    auto result = [&](std::vector<float>& r) {
      CK(hipStreamSynchronize(st));
      if (c.epi == EPI_SWIGLU) { std::vector<uint16_t> h((size_t)M * N / 2); CK(hipMemcpy(h.data(), out, h.size() * 2, hipMemcpyDeviceToHost)); r.resize(h.size()); for (size_t i = 0; i < h.size(); ++i) r[i] = bf2f(h[i]); }
      else { r.resize((size_t)M * N); CK(hipMemcpy(r.data(), y, r.size() * 4, hipMemcpyDeviceToHost)); }
    };
    auto run_check = [&](GemmLaunch L, std::vector<float>& r) {
      CK(hipMemcpyAsync(y, y0, (size_t)M * N * 4, hipMemcpyDeviceToDevice, st));
      CK(launch_gemm(L, st)); result(r);
    };
    auto timeit = [&](const GemmLaunch& base) {
      for (int w = 0; w < 2; ++w) for (int i = 0; i < NC; ++i) { GemmLaunch L = mk(i); L.force_S = base.force_S; L.force_R = base.force_R; L.force_ipw = base.force_ipw; L.force_W = base.force_W; L.force_KS = base.force_KS; CK(launch_gemm(L, st)); }
      CK(hipEventRecord(e0, st));
      const int reps = 4;
      for (int w = 0; w < reps; ++w) for (int i = 0; i < NC; ++i) { GemmLaunch L = mk(i); L.force_S = base.force_S; L.force_R = base.force_R; L.force_ipw = base.force_ipw; L.force_W = base.force_W; L.force_KS = base.force_KS; CK(launch_gemm(L, st)); }
      CK(hipEventRecord(e1, st)); CK(hipEventSynchronize(e1));
      float ms; CK(hipEventElapsedTime(&ms, e0, e1)); return ms * 1e3f / (reps * NC);
    };
    std::vector<float> ref; run_check(mk(0), ref);
    double refmax = 0; for (float v : ref) refmax = std::max(refmax, (double)fabsf(v));
    GemmPlan dp = plan_gemm(mk(0));
    const float tdef = timeit(mk(0));
    printf("== M=%d %s: tiles %d G %d (%.1f MB/launch, %d copies) default S=%d W=%d KS=%d R=%d grid=%d: %.2f us (%.0f GB/s)\n", M, c.name, c.tiles, c.G,
           (cb + sb) / 1e6, NC, dp.S, dp.waves, dp.KS, dp.R, dp.grid, tdef, (cb + sb) / (tdef * 1e3));
    fflush(stdout);
    struct Res { float t; GemmPlan p; int ipw; };
    std::vector<Res> res;
    for (int S : {1, 2, 3, 4, 5, 6, 8}) {
      if (S > c.G) continue;
      for (int W = 4; W <= 16; ++W) for (int KS = 1; KS <= W; ++KS) {
        if (W % KS) continue;
        for (int R : {2, 4, 8}) for (int ipw = 1; ipw <= 3; ++ipw) {
          GemmLaunch L = mk(0); L.force_S = S; L.force_W = W; L.force_KS = KS; L.force_R = R; L.force_ipw = ipw;
          GemmPlan p = plan_gemm(L);
          const int sbp = (c.G + S - 1) / S, Se = (c.G + sbp - 1) / sbp;
          if (p.S != Se || p.waves != W || p.KS != KS || p.R != R) continue;   // the forced plan did not fit
          const int T = W / KS, U = (c.tiles + T * ipw - 1) / (T * ipw);
          if (p.grid != Se * U) continue;
          if (p.grid > 1024) continue;
          std::vector<float> r; run_check(L, r);
          double md = 0; for (size_t i = 0; i < r.size(); ++i) md = std::max(md, (double)fabsf(r[i] - ref[i]) / (fabs(ref[i]) * 0.0079 + 1e-3 * refmax + 1e-3));
          if (!(md <= 1.0)) { printf("  MISMATCH S=%d W=%d KS=%d R=%d ipw=%d: max diff %g\n", S, W, KS, R, ipw, md); continue; }
          res.push_back({timeit(L), p, ipw});
        }
      }
    }
    std::sort(res.begin(), res.end(), [](const Res& a, const Res& b) { return a.t < b.t; });
    for (size_t i = 0; i < std::min<size_t>(6, res.size()); ++i) {
      const auto& q = res[i];
      printf("  %.2f us  S=%d sb=%d W=%d KS=%d R=%d ipw=%d grid=%d lds=%zu\n", q.t, q.p.S, q.p.sb_per_split, q.p.waves, q.p.KS, q.p.R, q.ipw, q.p.grid, q.p.lds);
    }
    printf("  (%zu plans)\n", res.size()); fflush(stdout);
    CK(hipFree(codes)); CK(hipFree(sm)); CK(hipFree(x)); CK(hipFree(ss)); CK(hipFree(A)); CK(hipFree(gain)); CK(hipFree(y)); CK(hipFree(y0)); CK(hipFree(out)); CK(hipFree(ssout));
  }
  return 0;
}
