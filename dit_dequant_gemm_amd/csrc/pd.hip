// Quantization-error tables and the PD-guided bit allocation ([WDQ] §3.2):
//   quant_sse_kernel   per-row sum of (w - w_hat32)^2 at every width 3..7 in
//                      one pass over W (the §3.1 quantizer, the same float32
//                      arithmetic as quantize_pack_kernel), float64 sums
//   sse_total_kernel   the rows' sums in a fixed order (deterministic)
//   ddg_pd_allocate    the host-side primal-dual search over those tables
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <system_error>
#include <thread>
#include <vector>

#include "ddg.h"
#include "ddg_launch.hpp"

namespace ddg {

constexpr int kSseWidths = 5;            // widths 3..7

// One workgroup of 1..4 waves per row; lane i takes chunks i, i+lanes, ...
// (32 weights each, the 4 chunks of a group in one quad).  The wave count is
// chosen on the host so that the last pass leaves few lanes idle.
template <bool F32_IN>
__global__ __launch_bounds__(256) void quant_sse_kernel(const void* __restrict__ w, int64_t k,
                                                       double* __restrict__ row_sse) {
  __shared__ double red[4][kSseWidths];
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const int lanes = blockDim.x;
  const int chunks = (int)(k / 32);
  double acc[kSseWidths] = {0.0, 0.0, 0.0, 0.0, 0.0};
  // whole quads per pass, so that the butterfly never mixes groups
  for (int c0 = 0; c0 < chunks; c0 += lanes) {
    const int c = c0 + lane;
    const bool valid = c < chunks;
    float v[32];
    if (valid) {
      if constexpr (F32_IN) {
        const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(w) + row * k + (int64_t)c * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const f32x4 t = src[i];
          v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
        }
      } else {
        const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(w) + row * k + (int64_t)c * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 t = src[i];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[8 * i + 2 * j] = bf16_bits_to_f32(t[j] & 0xFFFFu);
            v[8 * i + 2 * j + 1] = bf16_bits_to_f32(t[j] >> 16);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = 0.0f;
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
    a = __builtin_fmaxf(a, __shfl_xor(a, 1));
    a = __builtin_fmaxf(a, __shfl_xor(a, 2));
    const float a1 = a * 1.01f;
    [&]<int... J>(std::integer_sequence<int, J...>) {
      ([&] {
        constexpr int B = J + 3;
        constexpr float nh = (float)Bits<B>::n_half;
        const float step = (2.0f * a1) / (float)((1 << B) - 1);
        const bool zero_group = !(step != 0.0f);
        const bool fast = markstein_ok(step);
        float r[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) r[i] = v[i];
        quotients<32>(r, zero_group, fast, step, fast ? 1.0f / step : 0.0f);
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          float q = __builtin_rintf(r[i]);
          q = __builtin_fminf(__builtin_fmaxf(q, -nh), nh);
          const float wh = zero_group ? 0.0f : q * step;
          const double d = (double)v[i] - (double)wh;
          s = __builtin_fma(d, d, s);
        }
        acc[J] += s;
      }(), ...);
    }(std::make_integer_sequence<int, kSseWidths>{});
  }
  // workgroup sum: waves in order, lanes in a fixed butterfly
#pragma unroll
  for (int j = 0; j < kSseWidths; ++j) {
    double x = acc[j];
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    if ((lane & 63) == 0) red[lane >> 6][j] = x;
  }
  __syncthreads();
  if (lane < kSseWidths) {
    double x = red[0][lane];
    for (int wv = 1; wv < lanes / 64; ++wv) x += red[wv][lane];
    row_sse[row * kSseWidths + lane] = x;
  }
}

// totals[j] = sum over rows of row_sse[row][j], rows in order per lane
// stride, then a fixed butterfly.
__global__ __launch_bounds__(256) void sse_total_kernel(const double* __restrict__ row_sse, int64_t n,
                                                        double* __restrict__ total) {
  __shared__ double red[4][kSseWidths];
  const int lane = threadIdx.x;
  double acc[kSseWidths] = {0.0, 0.0, 0.0, 0.0, 0.0};
  for (int64_t r = lane; r < n; r += 256)
#pragma unroll
    for (int j = 0; j < kSseWidths; ++j) acc[j] += row_sse[r * kSseWidths + j];
#pragma unroll
  for (int j = 0; j < kSseWidths; ++j) {
    double x = acc[j];
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    if ((lane & 63) == 0) red[lane >> 6][j] = x;
  }
  __syncthreads();
  if (lane < kSseWidths) total[lane] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

hipError_t launch_quant_sse(const void* w, bool f32_in, int64_t n, int64_t k, double* row_sse,
                            double* total, hipStream_t stream) {
  if (n > 0) {
    // waves per row: the fewest lane slots over all passes, then the most waves
    const int64_t chunks = k / 32;
    int waves = 1;
    int64_t best = INT64_MAX;
    for (int wv = 1; wv <= 4; ++wv) {
      const int64_t slots = (chunks + 64 * wv - 1) / (64 * wv) * (64 * wv);
      if (slots <= best) { best = slots; waves = wv; }
    }
    if (f32_in)
      quant_sse_kernel<true><<<dim3((unsigned)n), dim3(64 * waves), 0, stream>>>(w, k, row_sse);
    else
      quant_sse_kernel<false><<<dim3((unsigned)n), dim3(64 * waves), 0, stream>>>(w, k, row_sse);
    if (hipError_t e = hipGetLastError()) return e;
  }
  sse_total_kernel<<<dim3(1), dim3(256), 0, stream>>>(row_sse, n, total);
  return hipGetLastError();
}

}  // namespace ddg

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
namespace {

constexpr double kPenalty = 1.0e4;       // the section's quadratic budget penalty
constexpr double kErrorPercent = 100.0;  // error term in percent of the uniform allocation's

// index of the candidate nearest x (the lower one on ties)
int nearest(const int* cand, int nc, double x) {
  int best = 0;
  double bd = std::fabs(x - cand[0]);
  for (int c = 1; c < nc; ++c) {
    const double d = std::fabs(x - cand[c]);
    if (d < bd) { bd = d; best = c; }
  }
  return best;
}

// Largest-remainder rounding within the budget: every tensor starts at the
// candidate at or below its continuous width; then, by decreasing fraction of
// the way to the next candidate (lower index first on ties), a tensor moves up
// one candidate when the added bits still fit in target * sum n.  idx gets the
// candidate index of every tensor.
void round_to_budget(const double* b, const int64_t* nparams, int n, const int* cand, int nc,
                     double budget, std::vector<int>& idx, std::vector<double>& frac,
                     std::vector<int>& order) {
  double spent = 0.0;
  for (int i = 0; i < n; ++i) {
    int j = 0;
    while (j + 1 < nc && (double)cand[j + 1] <= b[i]) ++j;
    idx[i] = j;
    frac[i] = j + 1 < nc ? (b[i] - cand[j]) / (double)(cand[j + 1] - cand[j]) : 0.0;
    spent += (double)nparams[i] * (double)cand[j];
  }
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return frac[x] > frac[y]; });
  for (int i : order) {
    if (!(frac[i] > 0.0)) continue;
    const double add = (double)nparams[i] * (double)(cand[idx[i] + 1] - cand[idx[i]]);
    if (spent + add <= budget) {
      ++idx[i];
      spent += add;
    }
  }
}

}  // namespace

extern "C" int ddg_quant_sse(const void* w, int w_dtype, int64_t n, int64_t k, double* row_sse,
                             double* total_sse, hipStream_t stream) {
  if (w_dtype != DDG_BF16 && w_dtype != DDG_F32) return DDG_ERR_ARG;
  if (n < 0 || n > DDG_SSE_ROWS_MAX || k <= 0 || k % DDG_GROUP || k > (INT64_C(1) << 31))
    return DDG_ERR_SHAPE;
  if (!total_sse) return DDG_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(total_sse) & 7) return DDG_ERR_ALIGN;
  if (n > 0) {
    if (!w || !row_sse) return DDG_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(w) & 15) || (reinterpret_cast<uintptr_t>(row_sse) & 7))
      return DDG_ERR_ALIGN;
  }
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return DDG_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return DDG_ERR_UNSUPPORTED;
  return ddg::launch_quant_sse(w, w_dtype == DDG_F32, n, k, row_sse, total_sse, stream) == hipSuccess
             ? DDG_OK
             : DDG_ERR_HIP;
}

extern "C" int ddg_pd_allocate(const double* sse, const int64_t* nparams, int n, const int* candidates,
                               int ncand, double target_bpw, const double* t_init, int restarts,
                               int iters, int* bits_out, double* info) {
  if (!sse || !nparams || !candidates || !t_init || !bits_out) return DDG_ERR_ARG;
  if (n < 1 || ncand < 2 || ncand > 8 || restarts < 1 || iters < 1) return DDG_ERR_SHAPE;
  for (int c = 1; c < ncand; ++c)
    if (candidates[c] <= candidates[c - 1]) return DDG_ERR_ARG;
  const double bmin = candidates[0], bmax = candidates[ncand - 1];
  if (!(target_bpw >= bmin && target_bpw <= bmax)) return DDG_ERR_ARG;
  for (int i = 0; i < n; ++i) {
    if (nparams[i] <= 0) return DDG_ERR_ARG;
    for (int c = 0; c < ncand; ++c)
      if (!(sse[(int64_t)i * ncand + c] >= 0.0) || !std::isfinite(sse[(int64_t)i * ncand + c]))
        return DDG_ERR_ARG;
  }
  // per-weight errors: the tensor's squared-error sum over its weight count
  std::vector<double> mse_v((size_t)n * ncand);
  for (int i = 0; i < n; ++i)
    for (int c = 0; c < ncand; ++c)
      mse_v[(size_t)i * ncand + c] = sse[(int64_t)i * ncand + c] / (double)nparams[i];
  const double* mse = mse_v.data();
  // weights of the tensors, and the error table in percent of the uniform
  // allocation at the candidate nearest the target
  double tot = 0.0;
  for (int i = 0; i < n; ++i) tot += (double)nparams[i];
  std::vector<double> wgt(n), m((size_t)n * ncand);
  double wsq = 0.0;
  for (int i = 0; i < n; ++i) {
    wgt[i] = (double)nparams[i] / tot;
    wsq += wgt[i] * wgt[i];
  }
  const int j0 = nearest(candidates, ncand, target_bpw);
  double ref = 0.0;
  for (int i = 0; i < n; ++i) ref += wgt[i] * mse[(int64_t)i * ncand + j0];
  for (size_t x = 0; x < m.size(); ++x)
    m[x] = ref > 0.0 ? kErrorPercent * mse[x] / ref : kErrorPercent * mse[x];
  // one step size for both updates: 1 / L, L the Lipschitz bound of the
  // budget penalty's gradient in the tensor parameters
  const double span = (bmax - bmin) / 4.0;
  const double step = 1.0 / (2.0 * kPenalty * span * span * wsq);
  const double budget = target_bpw * tot;

  // One restart: descent from its own starting point, then the rounding and
  // the exact score.  Restarts share nothing but the read-only tables.
  struct Outcome {
    int feasible = 0;
    double e = 0.0, p = 0.0;
    std::vector<int> bits;
  };
  std::vector<Outcome> out(restarts);
  auto run_restart = [&](int r) {
    std::vector<double> t(n), u(n), b(n), g(n), sw(ncand), frac(n);
    std::vector<int> idx(n), order(n);
    for (int i = 0; i < n; ++i) t[i] = t_init[(int64_t)r * n + i];
    double lam = 0.5;
    for (int it = 0; it < iters; ++it) {
      for (int i = 0; i < n; ++i) {
        u[i] = 1.0 / (1.0 + std::exp(-t[i]));
        b[i] = bmin + u[i] * (bmax - bmin);
      }
      const double temp = std::max(2.0 * (1.0 - (double)it / iters), 0.05);
      double bpw = 0.0;
      for (int i = 0; i < n; ++i) bpw += wgt[i] * b[i];
      const double gap = bpw - target_bpw;
      for (int i = 0; i < n; ++i) {
        // soft assignment of b[i] to the candidates, and the blended error
        double amax = -INFINITY;
        for (int c = 0; c < ncand; ++c) amax = std::max(amax, -std::fabs(b[i] - candidates[c]) / temp);
        double esum = 0.0;
        for (int c = 0; c < ncand; ++c) {
          sw[c] = std::exp(-std::fabs(b[i] - candidates[c]) / temp - amax);
          esum += sw[c];
        }
        double s = 0.0;
        for (int c = 0; c < ncand; ++c) { sw[c] /= esum; s += sw[c] * m[(size_t)i * ncand + c]; }
        double ds_db = 0.0;
        for (int c = 0; c < ncand; ++c) {
          const double dd = b[i] - candidates[c];
          const double sgn = dd > 0.0 ? 1.0 : (dd < 0.0 ? -1.0 : 0.0);
          ds_db += sw[c] * (m[(size_t)i * ncand + c] - s) * (-sgn / temp);
        }
        const double dl_db = wgt[i] * (ds_db + lam + 2.0 * kPenalty * gap);
        g[i] = dl_db * (bmax - bmin) * u[i] * (1.0 - u[i]);
      }
      for (int i = 0; i < n; ++i) t[i] = t[i] - step * g[i];
      lam = lam + step * gap;
    }
    // round within the budget and score the allocation exactly
    for (int i = 0; i < n; ++i) b[i] = bmin + (1.0 / (1.0 + std::exp(-t[i]))) * (bmax - bmin);
    round_to_budget(b.data(), nparams, n, candidates, ncand, budget, idx, frac, order);
    double e = 0.0, p = 0.0;
    for (int i = 0; i < n; ++i) {
      e += (double)nparams[i] * mse[(int64_t)i * ncand + idx[i]];
      p += (double)nparams[i] * (double)candidates[idx[i]];
    }
    Outcome& o = out[r];
    o.e = e / tot;
    o.p = p / tot;
    o.feasible = o.p <= target_bpw + 1e-9 ? 1 : 0;
    o.bits.resize(n);
    for (int i = 0; i < n; ++i) o.bits[i] = candidates[idx[i]];
  };
  // Restarts on up to 16 host threads, restart r on thread r mod T.  Each
  // restart's arithmetic is the same on any thread, so the result does not
  // depend on T; a thread that cannot be started leaves its restarts to the
  // calling thread.
  const int hw = (int)std::thread::hardware_concurrency();
  const int nthreads = std::max(1, std::min({restarts, hw > 0 ? hw : 1, 16}));
  auto run_stride = [&](int first) {
    for (int r = first; r < restarts; r += nthreads) run_restart(r);
  };
  std::vector<std::thread> pool;
  std::vector<int> orphaned;
  for (int w = 1; w < nthreads; ++w) {
    try {
      pool.emplace_back(run_stride, w);
    } catch (const std::system_error&) {
      orphaned.push_back(w);
    }
  }
  run_stride(0);
  for (int w : orphaned) run_stride(w);
  for (auto& th : pool) th.join();
  // the kept restart, compared in restart order
  int best = 0;
  for (int r = 1; r < restarts; ++r) {
    const Outcome &c = out[r], &k = out[best];
    bool better;
    if (c.feasible != k.feasible) better = c.feasible > k.feasible;
    else if (c.feasible) better = c.e < k.e || (c.e == k.e && c.p < k.p);
    else better = c.p < k.p || (c.p == k.p && c.e < k.e);
    if (better) best = r;
  }
  const std::vector<int>& best_bits = out[best].bits;
  const double best_e = out[best].e, best_p = out[best].p;
  const int best_restart = best;
  for (int i = 0; i < n; ++i) bits_out[i] = best_bits[i];
  if (info) { info[0] = best_e; info[1] = best_p; info[2] = best_restart; }
  return DDG_OK;
}
