// C ABI of libddg (declared in include/ddg.h): argument validation on the
// host, kernel choice, launch.  No allocation, no synchronization.
#include <algorithm>
#include <atomic>
#include <cstring>

#include "ddg.h"
#include "ddg_launch.hpp"

namespace {

constexpr int64_t kMaxDim = 2147483647;     // M, N fit a signed 32-bit int
constexpr int64_t kMaxK = INT64_C(1) << 20; // per-tile buffer ranges stay below 4 GiB
constexpr int kMaxDevices = 64;

// Per-device facts cached on first use: 0 unknown, 1 gfx950, -1 other.
std::atomic<int> g_dev_ok[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool bits_ok(int bits) { return bits >= 3 && bits <= 7; }

bool k_ok(int64_t k) { return k > 0 && k <= kMaxDim && k % DDG_GROUP == 0; }

// a * b without overflow past 2^62 (byte counts stay well inside int64).
bool mul_ok(int64_t a, int64_t b) { return a >= 0 && b >= 0 && (a == 0 || b <= (INT64_C(1) << 62) / a); }

// Current device: gfx950 check and compute-unit count.
int device_info(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DDG_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DDG_ERR_UNSUPPORTED;
  int ok = g_dev_ok[dev].load(std::memory_order_acquire);
  if (ok == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DDG_ERR_HIP;
    const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    ok = is950 ? 1 : -1;
    g_dev_ok[dev].store(ok, std::memory_order_release);
  }
  if (ok < 0) return DDG_ERR_UNSUPPORTED;
  *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return DDG_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DDG_OK : DDG_ERR_HIP; }

template <template <int> class F, typename... A>
hipError_t by_bits(int bits, A&&... args) {
  switch (bits) {
    case 3: return F<3>::run(args...);
    case 4: return F<4>::run(args...);
    case 5: return F<5>::run(args...);
    case 6: return F<6>::run(args...);
    case 7: return F<7>::run(args...);
  }
  return hipErrorInvalidValue;
}

template <int B>
struct QuantizeF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_quantize_pack<B>(a...); }
};
template <int B>
struct DequantizeF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_dequantize<B>(a...); }
};
template <int B>
struct LargeF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_gemm_large<B>(a...); }
};
template <int B>
struct SkinnyF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_gemm_skinny<B>(a...); }
};
template <int B>
struct SmallF {
  template <typename... A>
  static hipError_t run(A... a) { return ddg::launch_gemm_small<B>(a...); }
};

// Validation shared by the two GEMM entry points.
int check_gemm(const void* x, int64_t m, int64_t k, const uint8_t* packed, const float* scales,
               int bits, int64_t n, const void* y, int y_dtype) {
  if (!bits_ok(bits) || (y_dtype != DDG_BF16 && y_dtype != DDG_F32)) return DDG_ERR_ARG;
  if (m < 0 || m > kMaxDim || !k_ok(k) || k > kMaxK || n <= 0 || n > kMaxDim || n % 16)
    return DDG_ERR_SHAPE;
  if (!mul_ok(m, k) || !mul_ok(n, k) || !mul_ok(m, n)) return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!x || !packed || !scales || !y) return DDG_ERR_ARG;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 16) || !aligned(scales, 4))
    return DDG_ERR_ALIGN;
  return DDG_OK;
}

// Groups per wave chunk of the M <= 16 weight-streaming kernels for K = 128 g:
// the size (5, 4 or 3) that pads the busiest wave's share of K (ceil(g / 8)
// groups) with the fewest empty groups.
int skinny_chunk(int g) {
  const int per_wave = (g + 7) / 8;
  int kc = 5, waste = 1 << 30;
  for (int c = 5; c >= 3; --c) {
    const int w = (per_wave + c - 1) / c * c - per_wave;
    if (w < waste) { waste = w; kc = c; }
  }
  return kc;
}

// Kernel choice for the product; fills a.tiles_* for the large kernel.
hipError_t launch_product(ddg::GemmArgs& a, int bits, hipStream_t stream) {
  if (a.m <= 16) {
    // Wide outputs (at least 200 workgroups of 64 columns): the
    // weight-streaming kernel with an 8-way K split and X in registers.  Below
    // that it would either leave compute units idle or reload X (16 K bf16)
    // into too many workgroups; the LDS-ring kernel below is faster there.
    const int64_t nb = ((int64_t)a.n + 15) / 16;
    const int g = a.k / DDG_GROUP;
    if (nb / 4 >= 200) {
      int ncb = 4;
      int kc = skinny_chunk(g);
      // shrink until the weight buffers and the scale areas fit in LDS
      auto lds = [&] { return ddg::skinny_static_lds(bits, kc, ncb) + ddg::skinny_scale_lds(kc); };
      while (lds() > ddg::kLdsLimit && (ncb > 1 || kc > 3)) {
        if (ncb > 1) ncb /= 2; else --kc;
      }
      if (lds() <= ddg::kLdsLimit) return by_bits<SkinnyF>(bits, a, kc, ncb, stream);
    }
  }
  if (a.m <= 64) {
    const int rb = a.m <= 16 ? 1 : (a.m <= 32 ? 2 : 4);
    // Column waves x K-split waves per workgroup, from timings of the 16-,
    // 32- and 64-token products: four column waves where that still leaves
    // about 200+ workgroups (wide outputs; 16 tokens), two where 128+ remain,
    // else one column wave and an 8-way (16 tokens) or 4-way K split.
    const int64_t nb = ((int64_t)a.n + 15) / 16;
    int nc = 1, nk = rb == 1 ? 8 : 4;
    if (rb == 1 && nb / 4 >= 200) {
      nc = 4; nk = 2;
    } else if (nb / 2 >= 128) {
      nc = 2; nk = 2;
    }
    return by_bits<SmallF>(bits, a, rb, nc, nk, stream);
  }
  // large kernel: 256 x 256 tiles
  a.tiles_m = (a.m + ddg::kBM - 1) / ddg::kBM;
  a.tiles_n = (a.n + ddg::kBN - 1) / ddg::kBN;
  if ((int64_t)a.tiles_m * a.tiles_n > kMaxDim) return hipErrorInvalidValue;
  return by_bits<LargeF>(bits, a, stream);
}

}  // namespace

extern "C" {

int ddg_version(void) { return DDG_VERSION; }

const char* ddg_status_string(int status) {
  switch (status) {
    case DDG_OK: return "ok";
    case DDG_ERR_ARG: return "invalid argument (null pointer, dtype or bit width)";
    case DDG_ERR_SHAPE: return "invalid shape";
    case DDG_ERR_ALIGN: return "misaligned pointer";
    case DDG_ERR_WORKSPACE: return "workspace too small";
    case DDG_ERR_HIP: return "HIP launch or query failed";
    case DDG_ERR_UNSUPPORTED: return "current device is not gfx950";
  }
  return "unknown status";
}

int ddg_packed_bytes(int64_t n, int64_t k, int bits, int64_t* packed_bytes, int64_t* n_scales) {
  if (!packed_bytes || !n_scales || !bits_ok(bits)) return DDG_ERR_ARG;
  if (n < 0 || !k_ok(k) || !mul_ok(n, k) || !mul_ok(n * k, bits)) return DDG_ERR_SHAPE;
  *packed_bytes = n * k / 8 * bits;
  *n_scales = n * (k / DDG_GROUP);
  return DDG_OK;
}

int ddg_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int bits, uint8_t* packed,
                      float* scales, hipStream_t stream) {
  if (!bits_ok(bits) || (w_dtype != DDG_BF16 && w_dtype != DDG_F32)) return DDG_ERR_ARG;
  if (n < 0 || !k_ok(k) || !mul_ok(n, k) || !mul_ok(n * k, 4)) return DDG_ERR_SHAPE;
  if (n == 0) return DDG_OK;
  if (!w || !packed || !scales) return DDG_ERR_ARG;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 4)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  const int64_t n_chunks = n * k / 32;
  return hip_status(by_bits<QuantizeF>(bits, w, w_dtype == DDG_F32, n_chunks,
                                       reinterpret_cast<uint32_t*>(packed), scales, stream));
}

int ddg_dequantize(const uint8_t* packed, const float* scales, int bits, int64_t n, int64_t k,
                   void* w_out, hipStream_t stream) {
  if (!bits_ok(bits)) return DDG_ERR_ARG;
  if (n < 0 || !k_ok(k) || !mul_ok(n, k) || !mul_ok(n * k, 2)) return DDG_ERR_SHAPE;
  if (n == 0) return DDG_OK;
  if (!packed || !scales || !w_out) return DDG_ERR_ARG;
  if (!aligned(packed, 16) || !aligned(w_out, 16) || !aligned(scales, 4)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(by_bits<DequantizeF>(bits, packed, scales, n * k / 32, w_out, stream));
}

int ddg_dequant_gemm(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                     const float* scales, int bits, int64_t n, void* y, int y_dtype,
                     hipStream_t stream) {
  if (int st = check_gemm(x, m, k, packed, scales, bits, n, y, y_dtype)) return st;
  if (m == 0) return DDG_OK;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  ddg::GemmArgs a{};
  a.x = static_cast<const __bf16*>(x);
  a.packed = packed;
  a.scales = scales;
  a.y = y;
  a.t = nullptr;
  a.lora_up = nullptr;
  a.m = (int)m; a.n = (int)n; a.k = (int)k; a.r = 0;
  a.out_bf16 = y_dtype == DDG_BF16;
  return hip_status(launch_product(a, bits, stream));
}

int ddg_dequant_gemm_grouped(const ddg_gemm_desc* descs, int count, hipStream_t stream) {
  if (count < 0 || count > DDG_MAX_GROUPED) return DDG_ERR_SHAPE;
  if (count == 0) return DDG_OK;
  if (!descs) return DDG_ERR_ARG;
  int busy = 0;
  for (int i = 0; i < count; ++i) {
    const ddg_gemm_desc& d = descs[i];
    if (int st = check_gemm(d.x, d.m, d.k, d.packed, d.scales, d.bits, d.n, d.y, d.y_dtype))
      return st;
    busy += d.m > 0;
  }
  if (busy == 0) return DDG_OK;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  auto args_of = [](const ddg_gemm_desc& d) {
    ddg::GemmArgs a{};
    a.x = static_cast<const __bf16*>(d.x);
    a.packed = d.packed;
    a.scales = d.scales;
    a.y = d.y;
    a.t = nullptr;
    a.lora_up = nullptr;
    a.m = (int)d.m; a.n = (int)d.n; a.k = (int)d.k; a.r = 0;
    a.out_bf16 = d.y_dtype == DDG_BF16;
    return a;
  };
  // Products with M <= 16 share launches, longest workgroups first (their
  // work is about K * bits per workgroup) so that the short ones fill in.
  // Products with M > 64 share launches of the large kernel's tiles, deepest
  // K first; products with 16 < M <= 32 and 32 < M <= 64 share launches of
  // the small-M kernel's body (two column waves x a two-way K split), longest
  // workgroups first.
  int small[DDG_MAX_GROUPED], large[DDG_MAX_GROUPED], mid2[DDG_MAX_GROUPED], mid4[DDG_MAX_GROUPED];
  int n_small = 0, n_large = 0, n_mid2 = 0, n_mid4 = 0;
  for (int i = 0; i < count; ++i) {
    if (descs[i].m == 0) continue;
    if (descs[i].m <= 16) small[n_small++] = i;
    else if (descs[i].m <= 32) mid2[n_mid2++] = i;
    else if (descs[i].m <= 64) mid4[n_mid4++] = i;
    else large[n_large++] = i;
  }
  auto launch_mid = [&](int* list, int n_list, int rb) -> int {
    std::stable_sort(list, list + n_list, [&](int p, int q) {
      return descs[p].k * descs[p].bits > descs[q].k * descs[q].bits;
    });
    for (int s0 = 0; s0 < n_list; s0 += ddg::kMaxGroup) {
      ddg::GroupArgs ga{};
      ga.count = std::min(ddg::kMaxGroup, n_list - s0);
      ga.wg_start[0] = 0;
      for (int j = 0; j < ga.count; ++j) {
        const ddg_gemm_desc& d = descs[list[s0 + j]];
        ga.g[j] = args_of(d);
        ga.bits[j] = d.bits;
        const int64_t wgs = (d.n + 31) / 32;
        if (ga.wg_start[j] + wgs > kMaxDim) return DDG_ERR_SHAPE;
        ga.wg_start[j + 1] = ga.wg_start[j] + (int)wgs;
      }
      if (hipError_t e = ddg::launch_gemm_grouped_small(ga, rb, stream)) return hip_status(e);
    }
    return DDG_OK;
  };
  if (int st = launch_mid(mid2, n_mid2, 2)) return st;
  if (int st = launch_mid(mid4, n_mid4, 4)) return st;
  std::stable_sort(large, large + n_large, [&](int p, int q) { return descs[p].k > descs[q].k; });
  for (int s0 = 0; s0 < n_large; s0 += ddg::kMaxGroup) {
    ddg::GroupLargeArgs ga{};
    ga.count = std::min(ddg::kMaxGroup, n_large - s0);
    ga.tile_start[0] = 0;
    for (int j = 0; j < ga.count; ++j) {
      const ddg_gemm_desc& d = descs[large[s0 + j]];
      ga.g[j] = args_of(d);
      ga.g[j].tiles_m = (int)((d.m + ddg::kBM - 1) / ddg::kBM);
      ga.g[j].tiles_n = (int)((d.n + ddg::kBN - 1) / ddg::kBN);
      ga.bits[j] = d.bits;
      const int64_t tiles = (int64_t)ga.g[j].tiles_m * ga.g[j].tiles_n;
      if (ga.tile_start[j] + tiles > kMaxDim) return DDG_ERR_SHAPE;
      ga.tile_start[j + 1] = ga.tile_start[j] + (int)tiles;
    }
    if (hipError_t e = ddg::launch_gemm_grouped_large(ga, stream)) return hip_status(e);
  }
  std::stable_sort(small, small + n_small, [&](int p, int q) {
    return descs[p].k * descs[p].bits > descs[q].k * descs[q].bits;
  });
  for (int s0 = 0; s0 < n_small; s0 += ddg::kMaxGroup) {
    ddg::GroupArgs ga{};
    ga.count = std::min(ddg::kMaxGroup, n_small - s0);
    ga.wg_start[0] = 0;
    for (int j = 0; j < ga.count; ++j) {
      const ddg_gemm_desc& d = descs[small[s0 + j]];
      ga.g[j] = args_of(d);
      ga.bits[j] = d.bits;
      ga.kc[j] = skinny_chunk(d.k / DDG_GROUP);
      const int64_t wgs = (d.n + 16 * ddg::kGroupedNcb - 1) / (16 * ddg::kGroupedNcb);
      if (ga.wg_start[j] + wgs > kMaxDim) return DDG_ERR_SHAPE;
      ga.wg_start[j + 1] = ga.wg_start[j] + (int)wgs;
    }
    if (hipError_t e = ddg::launch_gemm_grouped(ga, stream)) return hip_status(e);
  }
  return DDG_OK;
}

int ddg_lowrank_workspace_bytes(int64_t m, int r, size_t* bytes) {
  if (!bytes) return DDG_ERR_ARG;
  if (m < 0 || m > kMaxDim || r < 8 || r > 128 || r % 8) return DDG_ERR_SHAPE;
  const int64_t raw = m * r * 2;
  *bytes = (size_t)((raw + 255) / 256 * 256);
  return DDG_OK;
}

int ddg_lowrank_fused_gemm(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                           const float* scales, int bits, int64_t n, const void* lora_down,
                           const void* lora_up, int r, void* y, int y_dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (int st = check_gemm(x, m, k, packed, scales, bits, n, y, y_dtype)) return st;
  if (r < 8 || r > 128 || r % 8) return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!lora_down || !lora_up || !workspace) return DDG_ERR_ARG;
  if (!aligned(lora_down, 16) || !aligned(lora_up, 16) || !aligned(workspace, 16))
    return DDG_ERR_ALIGN;
  size_t need = 0;
  ddg_lowrank_workspace_bytes(m, r, &need);
  if (workspace_bytes < need) return DDG_ERR_WORKSPACE;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  __bf16* t = static_cast<__bf16*>(workspace);
  if (hipError_t e = ddg::launch_lowrank_t(static_cast<const __bf16*>(x),
                                           static_cast<const __bf16*>(lora_down), t, (int)m,
                                           (int)k, r, stream))
    return hip_status(e);
  ddg::GemmArgs a{};
  a.x = static_cast<const __bf16*>(x);
  a.packed = packed;
  a.scales = scales;
  a.y = y;
  a.t = t;
  a.lora_up = static_cast<const __bf16*>(lora_up);
  a.m = (int)m; a.n = (int)n; a.k = (int)k; a.r = r;
  a.out_bf16 = y_dtype == DDG_BF16;
  return hip_status(launch_product(a, bits, stream));
}

int ddg_rpbh_rotate(const void* x, int x_dtype, int64_t n, int64_t d, const int32_t* perm,
                    const int8_t* signs, int h, void* out, int out_dtype, hipStream_t stream) {
  if ((x_dtype != DDG_BF16 && x_dtype != DDG_F32) || (out_dtype != DDG_BF16 && out_dtype != DDG_F32))
    return DDG_ERR_ARG;
  if (n < 0 || n > kMaxDim || d <= 0 || d % 64 || d > DDG_ROTATE_MAX_D || h < 2 ||
      h > DDG_ROTATE_MAX_H || (h & (h - 1)) || d % h || !mul_ok(n, d) || !mul_ok(n * d, 4))
    return DDG_ERR_SHAPE;
  if (n == 0) return DDG_OK;
  if (!x || !perm || !signs || !out) return DDG_ERR_ARG;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(perm, 4)) return DDG_ERR_ALIGN;
  // in place only as the very same buffer and type; otherwise no overlap
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x), oa = reinterpret_cast<uintptr_t>(out);
  const uintptr_t xb = xa + (uintptr_t)(n * d * (x_dtype == DDG_F32 ? 4 : 2));
  const uintptr_t ob = oa + (uintptr_t)(n * d * (out_dtype == DDG_F32 ? 4 : 2));
  const bool same = xa == oa && x_dtype == out_dtype;
  if (!same && xa < ob && oa < xb) return DDG_ERR_ARG;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(ddg::launch_rpbh_rotate(x, x_dtype == DDG_F32, n, (int)d, perm, signs, h, out,
                                            out_dtype == DDG_F32, cus, stream));
}

namespace {
// the 4-bit format in the low bits, DDG_FP4_POW2 and DDG_FP4_TILED the flags
constexpr int kFp4Flags = DDG_FP4_POW2 | DDG_FP4_TILED;
bool fp4_fmt_ok(int fmt) {
  const int f = fmt & ~kFp4Flags;
  return f >= DDG_FP4_E2M1 && f <= DDG_FP4_E1M2;
}
}  // namespace

int ddg_fp4_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int fmt, uint8_t* packed,
                          float* scales, hipStream_t stream) {
  if (!fp4_fmt_ok(fmt) || (w_dtype != DDG_BF16 && w_dtype != DDG_F32))
    return DDG_ERR_ARG;
  if (n < 0 || !k_ok(k) || !mul_ok(n, k) || !mul_ok(n * k, 4)) return DDG_ERR_SHAPE;
  if (n == 0) return DDG_OK;
  if (!w || !packed || !scales) return DDG_ERR_ARG;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 4)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(ddg::launch_fp4_quantize_pack(w, w_dtype == DDG_F32, n, (int)k, fmt & ~kFp4Flags,
                                                  (fmt & DDG_FP4_POW2) != 0, (fmt & DDG_FP4_TILED) != 0,
                                                  reinterpret_cast<uint32_t*>(packed), scales, stream));
}

int ddg_fp8_quantize_rows(const void* x, int64_t m, int64_t k, uint8_t* xq, float* xscales,
                          hipStream_t stream) {
  if (m < 0 || m > kMaxDim || !k_ok(k) || !mul_ok(m, k) || !mul_ok(m * k, 2)) return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!x || !xq || !xscales) return DDG_ERR_ARG;
  if (!aligned(x, 16) || !aligned(xq, 8) || !aligned(xscales, 4)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(ddg::launch_fp8_quantize_rows(static_cast<const uint16_t*>(x), m, (int)k, xq,
                                                  xscales, stream));
}

int ddg_fp6_quantize_rows(const void* x, int64_t m, int64_t k, int fmt6, uint8_t* xq, float* xscales,
                          hipStream_t stream) {
  if (fmt6 != DDG_FP6_E2M3 && fmt6 != DDG_FP6_E3M2) return DDG_ERR_ARG;
  if (m < 0 || m > kMaxDim || !k_ok(k) || !mul_ok(m + 31, k) || !mul_ok((m + 31) * k, 2)) return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!x || !xq || !xscales) return DDG_ERR_ARG;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xscales, 4)) return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  return hip_status(ddg::launch_fp6_quantize_rows(static_cast<const uint16_t*>(x), m, (int)k, fmt6, xq, xscales,
                                                  stream));
}

int ddg_w4a6_gemm(const uint8_t* xq, const float* xscales, int64_t m, int64_t k, int fmt6, const uint8_t* packed,
                  const float* wscales, int fmt, int64_t n, void* y, int y_dtype, hipStream_t stream) {
  if (fmt6 != DDG_FP6_E2M3 && fmt6 != DDG_FP6_E3M2) return DDG_ERR_ARG;
  if (!fp4_fmt_ok(fmt) || (y_dtype != DDG_BF16 && y_dtype != DDG_F32)) return DDG_ERR_ARG;
  if ((fmt & ~kFp4Flags) != DDG_FP4_E2M1 || !(fmt & DDG_FP4_TILED)) return DDG_ERR_ARG;   // tiled E2M1 only
  if (m < 0 || m > kMaxDim || !k_ok(k) || k > kMaxK || n <= 0 || n > kMaxDim || !mul_ok(m, n) ||
      !mul_ok(m * n, 4) || !mul_ok(n, k))
    return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!xq || !xscales || !packed || !wscales || !y) return DDG_ERR_ARG;
  if (!aligned(xq, 16) || !aligned(packed, 16) || !aligned(xscales, 4) || !aligned(wscales, 4) ||
      !aligned(y, y_dtype == DDG_F32 ? 4 : 2))
    return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  ddg::W4A8Args a{};
  a.xq = xq;
  a.xscales = xscales;
  a.packed = packed;
  a.wscales = wscales;
  a.y = y;
  a.m = (int)m; a.n = (int)n; a.k = (int)k;
  a.out_bf16 = y_dtype == DDG_BF16;
  return hip_status(ddg::launch_w4a6_gemm(a, fmt6, (fmt & DDG_FP4_POW2) != 0, stream));
}

int ddg_w4a8_gemm(const uint8_t* xq, const float* xscales, int64_t m, int64_t k, const uint8_t* packed,
                  const float* wscales, int fmt, int64_t n, void* y, int y_dtype, hipStream_t stream) {
  if (!fp4_fmt_ok(fmt) || (y_dtype != DDG_BF16 && y_dtype != DDG_F32))
    return DDG_ERR_ARG;
  if (m < 0 || m > kMaxDim || !k_ok(k) || k > kMaxK || n <= 0 || n > kMaxDim || !mul_ok(m, n) ||
      !mul_ok(m * n, 4) || !mul_ok(n, k))
    return DDG_ERR_SHAPE;
  if (m == 0) return DDG_OK;
  if (!xq || !xscales || !packed || !wscales || !y) return DDG_ERR_ARG;
  if (!aligned(xq, 16) || !aligned(packed, 16) || !aligned(xscales, 4) || !aligned(wscales, 4) ||
      !aligned(y, y_dtype == DDG_F32 ? 4 : 2))
    return DDG_ERR_ALIGN;
  int cus = 0;
  if (int st = device_info(&cus)) return st;
  ddg::W4A8Args a{};
  a.xq = xq;
  a.xscales = xscales;
  a.packed = packed;
  a.wscales = wscales;
  a.y = y;
  a.m = (int)m; a.n = (int)n; a.k = (int)k;
  a.out_bf16 = y_dtype == DDG_BF16;
  return hip_status(ddg::launch_w4a8_gemm(a, fmt & ~kFp4Flags, (fmt & DDG_FP4_POW2) != 0,
                                          (fmt & DDG_FP4_TILED) != 0, stream));
}

}  // extern "C"
