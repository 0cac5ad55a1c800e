// gauss_select.hip -- Gaussian-aware adaptive page selection: per-page key
// variance, the Gaussian moments of each page's logits, the threshold tau-hat
// of the distributional 1.5-entmax constraint, and the pages whose estimated
// maximum can cross it.
//
// EntmaxKV README "How it works": pages keep mean / std key statistics for the
// Gaussian-aware strategy; each page's scores are modelled as a Gaussian; the
// distributional entmax constraint is solved for tau-hat, with a page mixture
// for ALiBi heads and one Gaussian for NoPE heads; every page whose estimated
// maximum can cross tau-hat is kept, so the page count adapts.  The pages give
// no formulas; the readings taken here:
//   variance   population variance per dim over the page's valid rows,
//              around the fp32 page mean of pagestats_update;
//   moments    z = scale q.k (+ ALiBi bias slope (pos - (S - 1))):
//                mu  = scale q.mean (+ bias at the mean valid position),
//                var = scale^2 sum_d q_d^2 var_d (+ slope^2 (n^2 - 1) / 12,
//                      the variance of the bias over n consecutive positions);
//   tau-hat    with u = z / 2, the tau where the expected entmax mass
//              sum_tokens E[(u - tau)_+^2] is 1: each page adds
//              n_p E[(X - tau)_+^2] with X ~ N(mu_p / 2, var_p / 4)
//              (mixture), or the S tokens share the pooled N(mean, var)
//              (single);
//   estimate   est_p = mu_p + sqrt(var_p) sqrt(2 ln n_p) (the usual estimate
//              of the largest of n_p Gaussian draws; mu_p when n_p = 1);
//   selection  the reserved bos / eos pages and every other page with
//              est_p / 2 > tau-hat; at most k_cap pages (largest estimates,
//              ties to the lower index), at least one.  Qualifying pages are
//              exactly the ones of largest estimate, so this is the top-k
//              selection of skv_topk.h over the estimates with that budget.
//
// Arithmetic.  For X ~ N(m, s^2) and d = m - tau, a = d / s:
//   E[(X - tau)_+^2] = (d^2 + s^2) Phi(a) + d s phi(a),
//   E[(X - tau)_+]   = d Phi(a) + s phi(a)   (minus half the derivative).
// F(tau) = sum n_p E[(X_p - tau)_+^2] falls with tau, and tau0 =
// max_p (m_p - 1 / sqrt(n_p)) has F(tau0) >= 1 (Jensen); the root of F = 1 is
// found by safeguarded Newton steps on log F from tau0 (solve_tau).  The solve
// runs in fp64 (the two terms of the tail expectation cancel); the estimates
// and the comparison with tau-hat are fp32.
#include <math.h>

#include "skv_device.h"
#include "skv_host.h"
#include "skv_topk.h"

namespace {

constexpr int kWaves = 4;
constexpr int kIter = 2;
constexpr int kMaxNewton = 100;

// -------------------------------------------------------- page variance

// One block per (logical page, request), or per request for the tail page
// only.  A thread owns one 16-byte vector of the page's rows, as the
// statistics rebuild does.
__global__ __launch_bounds__(256) void page_var_kernel(
    const uint16_t* __restrict__ kv, int P, int row_vecs,
    const float* __restrict__ kmean, float* __restrict__ kvar,
    const int32_t* __restrict__ bt, int64_t bt_ld, const int32_t* __restrict__ seq_lens,
    int tail_only) {
  const int b = blockIdx.y;
  const int S = seq_lens[b];
  if (S <= 0) return;
  int64_t N = (static_cast<int64_t>(S) + P - 1) / P;
  if (N > bt_ld) N = bt_ld;
  const int64_t p = tail_only ? N - 1 : static_cast<int64_t>(blockIdx.x);
  if (p < 0 || p >= N) return;
  const int n = static_cast<int>(S - p * P < P ? S - p * P : P);
  const int64_t blk = bt[static_cast<int64_t>(b) * bt_ld + p];
  const int64_t row_elems = static_cast<int64_t>(row_vecs) * 8;
  const uint16_t* page = kv + blk * P * row_elems;
  const float inv = 1.0f / static_cast<float>(n);
  for (int v = threadIdx.x; v < row_vecs; v += blockDim.x) {
    const float4 m0 = *reinterpret_cast<const float4*>(kmean + blk * row_elems + v * 8);
    const float4 m1 = *reinterpret_cast<const float4*>(kmean + blk * row_elems + v * 8 + 4);
    const float m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    float ss[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ss[i] = 0.0f;
    for (int t = 0; t < n; ++t) {
      float x[8];
      skv::unpack8(*reinterpret_cast<const uint4*>(page + t * row_elems + v * 8), x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = x[i] - m[i];
        ss[i] = fmaf(d, d, ss[i]);
      }
    }
    float4* dst = reinterpret_cast<float4*>(kvar + blk * row_elems + v * 8);
    dst[0] = make_float4(ss[0] * inv, ss[1] * inv, ss[2] * inv, ss[3] * inv);
    dst[1] = make_float4(ss[4] * inv, ss[5] * inv, ss[6] * inv, ss[7] * inv);
  }
}

// -------------------------------------------------------- logit moments

// Mapping as the page score: one block per (tile of pages, kv head x slice
// of up to GS query heads, request); D/8 lanes per page-head with 16-byte
// loads of the mean and variance rows (512 + 512 bytes at D = 128), read once
// for the slice, whose scaled query rows sit in LDS.
template <int D, int GS>
__global__ __launch_bounds__(256) void gauss_moments_kernel(
    const float* __restrict__ q, int H_q, int H_kv, int G,
    const float* __restrict__ kmean, const float* __restrict__ kvar,
    const int32_t* __restrict__ bt, int64_t bt_ld, const int32_t* __restrict__ seq_lens,
    int P, float scale, const float* __restrict__ alibi, float* __restrict__ mu,
    float* __restrict__ var, int64_t ld) {
  constexpr int LPR = D / 8;
  constexpr int PPW = 64 / LPR;
  constexpr int TILE = kIter * kWaves * PPW;
  const int b = blockIdx.z;
  const int nslices = (G + GS - 1) / GS;
  const int h = blockIdx.x / nslices;
  const int g0 = (blockIdx.x % nslices) * GS;
  const int S = seq_lens[b];
  int64_t N = (static_cast<int64_t>(S) + P - 1) / P;
  if (N > bt_ld) N = bt_ld;
  const int64_t p0 = static_cast<int64_t>(blockIdx.y) * TILE;
  if (p0 >= N) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane / LPR;
  const int c = lane % LPR;
  const float slope = alibi != nullptr && c < GS && g0 + c < G ? alibi[h * G + g0 + c] : 0.0f;

  const int32_t* btr = bt + static_cast<int64_t>(b) * bt_ld;
  float4 me[kIter][2], va[kIter][2];
  int64_t pg[kIter];
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    pg[it] = p0 + (it * kWaves + wave) * PPW + sub;
    const int64_t blk = btr[pg[it] < N ? pg[it] : p0];
    const int64_t off = (blk * H_kv + h) * D + c * 8;
    me[it][0] = *reinterpret_cast<const float4*>(kmean + off);
    me[it][1] = *reinterpret_cast<const float4*>(kmean + off + 4);
    va[it][0] = *reinterpret_cast<const float4*>(kvar + off);
    va[it][1] = *reinterpret_cast<const float4*>(kvar + off + 4);
  }
  __shared__ __align__(16) float qs[GS][D];          // scale * q
  for (int i = threadIdx.x; i < GS * D; i += blockDim.x) {
    const int g = i / D, d = i % D;
    qs[g][d] = g0 + g < G
                   ? scale * q[(static_cast<int64_t>(b) * H_q + h * G + g0 + g) * D + d]
                   : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const float m8[8] = {me[it][0].x, me[it][0].y, me[it][0].z, me[it][0].w,
                         me[it][1].x, me[it][1].y, me[it][1].z, me[it][1].w};
    const float v8[8] = {va[it][0].x, va[it][0].y, va[it][0].z, va[it][0].w,
                         va[it][1].x, va[it][1].y, va[it][1].z, va[it][1].w};
    float my_mu = 0.0f, my_var = 0.0f;
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      const float4 qa = *reinterpret_cast<const float4*>(&qs[g][c * 8]);
      const float4 qb = *reinterpret_cast<const float4*>(&qs[g][c * 8 + 4]);
      const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s1 = fmaf(qv[i], m8[i], s1);
        s2 = fmaf(qv[i] * qv[i], v8[i], s2);
      }
      s1 = skv::group_sum<LPR>(s1);
      s2 = skv::group_sum<LPR>(s2);
      if (c == g) { my_mu = s1; my_var = s2; }
    }
    if (pg[it] < N && c < GS && g0 + c < G) {
      if (alibi != nullptr) {
        const int64_t nn = static_cast<int64_t>(S) - pg[it] * P;
        const float n = static_cast<float>(nn < P ? nn : P);
        // integer offset of the page's first row from the query, exact in fp32
        const float first = static_cast<float>(pg[it] * P - (S - 1));
        my_mu = fmaf(slope, first + 0.5f * (n - 1.0f), my_mu);
        my_var = fmaf(slope * slope, (n * n - 1.0f) * (1.0f / 12.0f), my_var);
      }
      const int64_t o = (static_cast<int64_t>(b) * H_q + h * G + g0 + c) * ld + pg[it];
      mu[o] = my_mu;
      var[o] = my_var;
    }
  }
}

// -------------------------------------------------------- tau-hat + select

// fp64 wave reductions: DPP moves of both 32-bit halves inside each 16-lane
// row (no LDS permutes), then the four row results read into scalars; every
// lane gets the same value.
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(x));
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u & 0xffffffffull), CTRL,
                                             0xF, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, 0xF, 0xF,
                                             true);
  return __longlong_as_double(static_cast<long long>(
      (static_cast<unsigned long long>(static_cast<unsigned int>(hi)) << 32) |
      static_cast<unsigned int>(lo)));
}

__device__ __forceinline__ double lane_d(double x, int l) {
  const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(x));
  const unsigned int lo = __builtin_amdgcn_readlane(static_cast<int>(u & 0xffffffffull), l);
  const unsigned int hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), l);
  return __longlong_as_double(static_cast<long long>(
      (static_cast<unsigned long long>(hi) << 32) | lo));
}

__device__ __forceinline__ double wave_sum_d(double x) {
  x += dpp_d<0xB1>(x);
  x += dpp_d<0x4E>(x);
  x += dpp_d<0x141>(x);
  x += dpp_d<0x140>(x);
  return (lane_d(x, 0) + lane_d(x, 16)) + (lane_d(x, 32) + lane_d(x, 48));
}

__device__ __forceinline__ double wave_max_d(double x) {
  x = fmax(x, dpp_d<0xB1>(x));
  x = fmax(x, dpp_d<0x4E>(x));
  x = fmax(x, dpp_d<0x141>(x));
  x = fmax(x, dpp_d<0x140>(x));
  return fmax(fmax(lane_d(x, 0), lane_d(x, 16)), fmax(lane_d(x, 32), lane_d(x, 48)));
}

// Sums of two doubles over the block; red holds 2 * (waves) doubles.
__device__ __forceinline__ void block_sum2_d(double& x, double& y, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  x = wave_sum_d(x);
  y = wave_sum_d(y);
  if (lane == 0) { red[2 * wave] = x; red[2 * wave + 1] = y; }
  __syncthreads();
  x = 0.0; y = 0.0;
  for (int w = 0; w < nw; ++w) { x += red[2 * w]; y += red[2 * w + 1]; }
  __syncthreads();
}

__device__ __forceinline__ double block_max_d(double x, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  x = wave_max_d(x);
  if (lane == 0) red[wave] = x;
  __syncthreads();
  double t = -INFINITY;
  for (int w = 0; w < nw; ++w) t = fmax(t, red[w]);
  __syncthreads();
  return t;
}

// (E[(X - tau)_+^2], E[(X - tau)_+]) for X ~ N(m, s^2).  Beyond 9 standard
// deviations the Gaussian tail (below 1e-18 of the scale) is dropped: a page
// far below tau adds nothing, one far above adds d^2 + s^2 and d.
__device__ __forceinline__ void gauss_excess(double m, double s, double tau, double& e2,
                                             double& e1) {
  const double d = m - tau;
  if (!(s > 0.0) || d >= 9.0 * s) {
    const double dp = d > 0.0 ? d : 0.0;
    e2 = dp * dp + (dp > 0.0 ? s * s : 0.0);
    e1 = dp;
    return;
  }
  if (d <= -9.0 * s) { e2 = 0.0; e1 = 0.0; return; }
  const double a = d / s;
  const double Phi = 0.5 * erfc(-a * 0.70710678118654752440);     // 1 / sqrt(2)
  const double phi = exp(-0.5 * a * a) * 0.39894228040143267794;  // 1 / sqrt(2 pi)
  e2 = (d * d + s * s) * Phi + d * s * phi;
  e1 = d * Phi + s * phi;
  if (e2 < 0.0) e2 = 0.0;
  if (e1 < 0.0) e1 = 0.0;
}

// A first guess of the single-Gaussian root: with a = (m - tau) / s the
// constraint reads S s^2 psi(a) = 1, psi(a) = (1 + a^2) Phi(a) + a phi(a),
// which behaves as 1 + a^2 for a >= 1, runs from 0.5 to about 1.9 on [0, 1],
// and as 2 phi(a) / |a|^3 far below 0.  Newton steps correct the guess; it
// only saves steps, and it never lies below the Jensen start.
__device__ __forceinline__ double start_single(double m, double s, double S) {
  if (!(s > 0.0)) return m - 1.0 / sqrt(S);
  const double r = 1.0 / (S * s * s);
  double a;
  if (r >= 2.0) {
    a = sqrt(r - 1.0);
  } else if (r >= 0.5) {
    a = (r - 0.5) / 1.42;
  } else {
    // 2 phi(x) / x^3 = r  ->  x^2 = 2 ln(2 / (sqrt(2 pi) r)) - 6 ln x
    const double c = 2.0 * log(0.79788456080286535588 / r);   // 2 / sqrt(2 pi)
    double x = sqrt(c > 1.0 ? c : 1.0);
    for (int k = 0; k < 3; ++k) {
      const double x2 = c - 6.0 * log(x > 1.0 ? x : 1.0);
      x = sqrt(x2 > 0.0 ? x2 : 0.0);
    }
    a = -x;
  }
  const double t = m - a * s;
  const double lo = m - 1.0 / sqrt(S);
  return t > lo ? t : lo;
}

// Root of F(tau) = 1, F(tau) = sum n E[(X - tau)_+^2] with F' = -2 sum n
// E[(X - tau)_+] (eval returns F and that sum), from lo with F(lo) >= 1.
// Newton steps on log F: for one Gaussian log F is concave (the threshold
// moments of a log-concave density are log-concave), so after the first
// step the iterates fall monotonically onto the root in a few steps; a
// bracket [lo, hi] with F(lo) >= 1 > F(hi) catches anything else (a
// mixture, an underflowed F) with a bisection.  The result is uniform across
// the callers when eval is.
template <class Eval>
__device__ double solve_tau(double lo, double start, Eval eval) {
  double hi = INFINITY, tau = start > lo ? start : lo;
  for (int it = 0; it < kMaxNewton; ++it) {
    double F, G;
    eval(tau, F, G);
    if (F >= 1.0) lo = tau; else hi = tau;
    double next = (F > 0.0 && G > 0.0) ? tau + log(F) * F / (2.0 * G) : NAN;
    if (!(next >= lo && next <= hi))
      next = hi < INFINITY ? 0.5 * (lo + hi) : lo + fmax(1.0, fabs(lo));
    if (!(fabs(next - tau) > 1e-13 * fmax(1.0, fabs(tau)))) return next;
    tau = next;
  }
  return tau;
}

// Pages a mixture solve keeps in LDS: those whose Gaussian reaches within 9
// standard deviations of the lower start tau0 (tau-hat never goes below it,
// so the rest add nothing at any step).  Rows with more read the whole row
// from memory at every step instead.
constexpr int kAliveCap = 2048;

// One block per (request, query head) row; entry p is handled by thread
// p mod BLOCK in every pass.
template <int BLOCK, int ITEMS>
__global__ __launch_bounds__(BLOCK) void gauss_select_kernel(
    const float* __restrict__ mu, const float* __restrict__ var, int64_t ld, int H_q,
    const int32_t* __restrict__ seq_lens, int P, const int32_t* __restrict__ bt,
    int64_t bt_ld, int mixture, int bos, int eos, int k_cap, float* __restrict__ tau_out,
    float* est, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt,
    int32_t* __restrict__ sel_blk) {
  __shared__ double red[2 * (BLOCK / 64)];
  __shared__ int ired[BLOCK / 64 + 1];
  __shared__ float al_m[kAliveCap], al_v[kAliveCap], al_n[kAliveCap];
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>(row / H_q);
  const int S = seq_lens[b];
  int64_t N64 = S > 0 ? (static_cast<int64_t>(S) + P - 1) / P : 0;
  if (N64 > bt_ld) N64 = bt_ld;
  const int N = static_cast<int>(N64);
  const int tid = threadIdx.x;
  const float* mr = mu + row * ld;
  const float* vr = var + row * ld;
  float* er = est + row * ld;
  auto rows_of = [&](int p) { return S - p * P < P ? S - p * P : P; };
  // The row (8 bytes a page) is read from cache by each pass (strided,
  // coalesced): registers stay free for the fp64 tail expectations.
  auto m_of = [&](int p) { return 0.5 * static_cast<double>(mr[p]); };
  auto s_of = [&](int p) { return 0.5 * sqrt(static_cast<double>(fmaxf(vr[p], 0.0f))); };

  __shared__ double s_tau;
  double tau = -INFINITY;
  if (N > 0) {
    if (mixture) {
      double t0 = -INFINITY;
      for (int p = tid; p < N; p += BLOCK)
        t0 = fmax(t0, m_of(p) - 1.0 / sqrt(static_cast<double>(rows_of(p))));
      t0 = block_max_d(t0, red);
      // the pages that can matter at any tau >= t0 go to an LDS list
      auto alive = [&](int p) { return m_of(p) + 9.0 * s_of(p) > t0; };
      int na = 0;
      for (int p = tid; p < N; p += BLOCK) na += alive(p) ? 1 : 0;
      int total;
      int pos = skv::block_exclusive_scan(na, &total, ired);
      const bool in_lds = total <= kAliveCap;
      if (in_lds)
        for (int p = tid; p < N; p += BLOCK)
          if (alive(p)) {
            al_m[pos] = mr[p];
            al_v[pos] = fmaxf(vr[p], 0.0f);
            al_n[pos] = static_cast<float>(rows_of(p));
            ++pos;
          }
      __syncthreads();
      const int count = in_lds ? total : N;
      tau = solve_tau(t0, t0, [&](double t, double& F, double& G) {
        double f = 0.0, g = 0.0, e2, e1;
        for (int j = tid; j < count; j += BLOCK) {
          // the LDS list, or the whole row from memory
          const float mj = in_lds ? al_m[j] : mr[j];
          const float vj = in_lds ? al_v[j] : fmaxf(vr[j], 0.0f);
          const double nj = in_lds ? static_cast<double>(al_n[j])
                                   : static_cast<double>(rows_of(j));
          gauss_excess(0.5 * static_cast<double>(mj), 0.5 * sqrt(static_cast<double>(vj)), t,
                       e2, e1);
          f = fma(nj, e2, f);
          g = fma(nj, e1, g);
        }
        block_sum2_d(f, g, red);
        F = f;
        G = g;
      });
    } else {
      // pooled mean, then the pooled variance around it (law of total
      // variance, no cancellation)
      double sn = 0.0, sm = 0.0;
      for (int p = tid; p < N; p += BLOCK) {
        const double n = static_cast<double>(rows_of(p));
        sn += n;
        sm = fma(n, static_cast<double>(mr[p]), sm);
      }
      block_sum2_d(sn, sm, red);
      const double Sd = sn;                             // valid tokens of the N pages
      const double gm = sm / Sd;
      double sv = 0.0, unused = 0.0;
      for (int p = tid; p < N; p += BLOCK) {
        const double dm = static_cast<double>(mr[p]) - gm;
        sv = fma(static_cast<double>(rows_of(p)),
                 static_cast<double>(fmaxf(vr[p], 0.0f)) + dm * dm, sv);
      }
      block_sum2_d(sv, unused, red);
      // one scalar solve: wave 0 runs it, the block reads the result
      if (tid < 64) {
        const double m = 0.5 * gm, s = 0.5 * sqrt(sv / Sd);
        const double t = solve_tau(m - 1.0 / sqrt(Sd), start_single(m, s, Sd),
                                   [&](double t, double& F, double& G) {
          double e2, e1;
          gauss_excess(m, s, t, e2, e1);
          F = Sd * e2;
          G = Sd * e1;
        });
        if (tid == 0) s_tau = t;
      }
      __syncthreads();
      tau = s_tau;
    }
  }
  const float tau_f = static_cast<float>(tau);

  // estimated maxima, and the count of qualifying pages between the reserved
  const int lo = bos < N ? bos : N;
  int hi = N - eos > 0 ? N - eos : 0;
  if (hi < lo) hi = lo;
  int qual = 0;
  for (int p = tid; p < N; p += BLOCK) {
    const int n = rows_of(p);
    const float c = n > 1 ? sqrtf(2.0f * logf(static_cast<float>(n))) : 0.0f;
    const float e = fmaf(sqrtf(fmaxf(vr[p], 0.0f)), c, mr[p]);
    er[p] = e;
    if (p >= lo && p < hi && 0.5f * e > tau_f) ++qual;
  }
  {
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) qual += __shfl_xor(qual, o);
    if (lane == 0) ired[wave] = qual;
    __syncthreads();                  // also orders the estimate stores
    qual = 0;
    for (int w = 0; w < BLOCK / 64; ++w) qual += ired[w];
  }
  const int nres = N - (hi - lo);
  int budget = qual + nres;
  if (budget > k_cap) budget = k_cap;
  if (budget < 1) budget = 1;
  const bool aligned = ((ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(est) & 15) == 0);
  const int total = skv::topk_row<BLOCK, ITEMS>(
      er, aligned, N, budget, 0.0, bos, eos,
      sel_blk != nullptr ? bt + static_cast<int64_t>(b) * bt_ld : nullptr, bt_ld,
      sel_idx + row * k_cap, sel_blk != nullptr ? sel_blk + row * k_cap : nullptr, k_cap);
  if (tid == 0) {
    sel_cnt[row] = total;
    if (tau_out != nullptr) tau_out[row] = tau_f;
  }
}

template <int BLOCK, int ITEMS>
void launch_select(int64_t rows, hipStream_t stream, const float* mu, const float* var,
                   int64_t ld, int H_q, const int32_t* seq_lens, int P, const int32_t* bt,
                   int64_t bt_ld, int mixture, int bos, int eos, int k_cap, float* tau,
                   float* est, int32_t* sel_idx, int32_t* sel_cnt, int32_t* sel_blk) {
  hipLaunchKernelGGL((gauss_select_kernel<BLOCK, ITEMS>), dim3(static_cast<unsigned>(rows)),
                     dim3(BLOCK), 0, stream, mu, var, ld, H_q, seq_lens, P, bt, bt_ld,
                     mixture, bos, eos, k_cap, tau, est, sel_idx, sel_cnt, sel_blk);
}

}  // namespace

extern "C" int page_var_update(const uint16_t* kv_cache, int64_t num_blocks, int page_size,
                               int H_kv, int D, const float* k_mean, float* k_var,
                               const int32_t* block_table, int64_t bt_ld,
                               const int32_t* seq_lens, int B, int tail_only,
                               hipStream_t stream) {
  SKV_REQUIRE(B >= 0 && H_kv > 0 && num_blocks > 0 && bt_ld > 0,
              "page_var_update: need B >= 0, H_kv > 0, num_blocks > 0, bt_ld > 0");
  SKV_REQUIRE(D == 64 || D == 128, "page_var_update: D must be 64 or 128 (got %d)", D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "page_var_update: page_size must be 1, 2, 4, 8 or 16 (got %d)", page_size);
  SKV_REQUIRE(bt_ld <= 0x7fffffff && B <= 65535, "page_var_update: grid too large");
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR(kv_cache);
  SKV_REQUIRE_PTR(k_mean);
  SKV_REQUIRE_PTR(k_var);
  SKV_REQUIRE_PTR(block_table);
  SKV_REQUIRE_PTR(seq_lens);
  const int row_vecs = H_kv * D / 8;
  const int threads = row_vecs >= 256 ? 256 : ((row_vecs + 63) / 64) * 64;
  const dim3 grid(tail_only ? 1u : static_cast<unsigned>(bt_ld), static_cast<unsigned>(B));
  hipLaunchKernelGGL(page_var_kernel, grid, dim3(threads), 0, stream, kv_cache, page_size,
                     row_vecs, k_mean, k_var, block_table, bt_ld, seq_lens, tail_only ? 1 : 0);
  SKV_CHECK_LAUNCH();
}

extern "C" int gauss_moments(const float* q, int B, int H_q, int H_kv, int D,
                             const float* k_mean, const float* k_var,
                             const int32_t* block_table, int64_t bt_ld,
                             const int32_t* seq_lens, int page_size, float scale,
                             const float* alibi_slopes, float* mu, float* var, int64_t ld,
                             hipStream_t stream) {
  SKV_REQUIRE(B >= 0 && H_kv > 0 && H_q > 0 && H_q % H_kv == 0,
              "gauss_moments: need H_q a positive multiple of H_kv (H_q=%d, H_kv=%d)", H_q,
              H_kv);
  const int G = H_q / H_kv;
  SKV_REQUIRE(G <= 16, "gauss_moments: group size %d > 16", G);
  SKV_REQUIRE(D == 64 || D == 128, "gauss_moments: D must be 64 or 128 (got %d)", D);
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "gauss_moments: page_size must be 1, 2, 4, 8 or 16 (got %d)", page_size);
  SKV_REQUIRE(bt_ld > 0 && ld >= bt_ld, "gauss_moments: need bt_ld > 0 and ld >= bt_ld");
  SKV_REQUIRE(scale > 0.0f, "gauss_moments: scale must be > 0");
  SKV_REQUIRE(B <= 65535, "gauss_moments: grid too large");
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR(q);
  SKV_REQUIRE_PTR(k_mean);
  SKV_REQUIRE_PTR(k_var);
  SKV_REQUIRE_PTR(block_table);
  SKV_REQUIRE_PTR(seq_lens);
  SKV_REQUIRE_PTR(mu);
  SKV_REQUIRE_PTR(var);
  const int GS = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
  const int slices = (G + GS - 1) / GS;
  const int tile = kIter * kWaves * (64 / (D / 8));
  const int64_t tiles = (bt_ld + tile - 1) / tile;
  SKV_REQUIRE(tiles <= 65535, "gauss_moments: bt_ld %lld too long", (long long)bt_ld);
  const dim3 grid(static_cast<unsigned>(H_kv * slices), static_cast<unsigned>(tiles),
                  static_cast<unsigned>(B));
#define SKV_MOM(DD, GG)                                                                  \
  hipLaunchKernelGGL((gauss_moments_kernel<DD, GG>), grid, dim3(256), 0, stream, q, H_q, \
                     H_kv, G, k_mean, k_var, block_table, bt_ld, seq_lens, page_size,    \
                     scale, alibi_slopes, mu, var, ld)
  if (D == 128) {
    if (GS == 1) SKV_MOM(128, 1); else if (GS == 2) SKV_MOM(128, 2);
    else if (GS == 4) SKV_MOM(128, 4); else SKV_MOM(128, 8);
  } else {
    if (GS == 1) SKV_MOM(64, 1); else if (GS == 2) SKV_MOM(64, 2);
    else if (GS == 4) SKV_MOM(64, 4); else SKV_MOM(64, 8);
  }
#undef SKV_MOM
  SKV_CHECK_LAUNCH();
}

extern "C" int gauss_select(const float* mu, const float* var, int64_t ld, int B, int H_q,
                            const int32_t* seq_lens, int page_size,
                            const int32_t* block_table, int64_t bt_ld, int mixture,
                            int reserved_bos, int reserved_eos, int k_cap, float* tau,
                            float* est, int32_t* sel_idx, int32_t* sel_cnt,
                            int32_t* sel_blk, hipStream_t stream) {
  SKV_REQUIRE(B >= 0 && H_q > 0, "gauss_select: need B >= 0 and H_q > 0");
  SKV_REQUIRE(skv_supported_page_size(page_size),
              "gauss_select: page_size must be 1, 2, 4, 8 or 16 (got %d)", page_size);
  SKV_REQUIRE(bt_ld > 0 && bt_ld <= 32768 && ld >= bt_ld,
              "gauss_select: need 0 < bt_ld <= 32768 and ld >= bt_ld");
  SKV_REQUIRE(reserved_bos >= 0 && reserved_eos >= 0,
              "gauss_select: reserved_bos / reserved_eos must be >= 0");
  SKV_REQUIRE(k_cap >= 1, "gauss_select: k_cap must be >= 1");
  int64_t nres = static_cast<int64_t>(reserved_bos) + reserved_eos;
  if (nres > bt_ld) nres = bt_ld;
  SKV_REQUIRE(k_cap >= nres, "gauss_select: k_cap %d < reserved pages %lld", k_cap,
              (long long)nres);
  // no rows: nothing is read or written, so no pointer is needed
  if (B == 0) { skv::clear_error(); return SKV_OK; }
  SKV_REQUIRE_PTR(mu);
  SKV_REQUIRE_PTR(var);
  SKV_REQUIRE_PTR(seq_lens);
  SKV_REQUIRE_PTR(block_table);
  SKV_REQUIRE_PTR(est);
  SKV_REQUIRE_PTR(sel_idx);
  SKV_REQUIRE_PTR(sel_cnt);
  const int64_t rows = static_cast<int64_t>(B) * H_q;
  SKV_REQUIRE(rows <= 0x7fffffff, "gauss_select: too many rows");
  const int mix = mixture ? 1 : 0;
#define SKV_GSEL(BL, IT)                                                               \
  launch_select<BL, IT>(rows, stream, mu, var, ld, H_q, seq_lens, page_size,           \
                        block_table, bt_ld, mix, reserved_bos, reserved_eos, k_cap, tau, \
                        est, sel_idx, sel_cnt, sel_blk)
  if (rows < 1024) {
    // few rows, each latency-bound: wide blocks, short loops per thread
    if (bt_ld <= 1024) SKV_GSEL(256, 4);
    else if (bt_ld <= 2048) SKV_GSEL(512, 4);
    else if (bt_ld <= 4096) SKV_GSEL(1024, 4);
    else if (bt_ld <= 8192) SKV_GSEL(1024, 8);
    else if (bt_ld <= 16384) SKV_GSEL(1024, 16);
    else SKV_GSEL(1024, 32);
  } else {
    // rows enough to fill the chip: 256-thread blocks, several per CU
    if (bt_ld <= 1024) SKV_GSEL(256, 4);
    else if (bt_ld <= 2048) SKV_GSEL(256, 8);
    else if (bt_ld <= 4096) SKV_GSEL(256, 16);
    else if (bt_ld <= 8192) SKV_GSEL(512, 16);
    else if (bt_ld <= 16384) SKV_GSEL(1024, 16);
    else SKV_GSEL(1024, 32);
  }
#undef SKV_GSEL
  SKV_CHECK_LAUNCH();
}
